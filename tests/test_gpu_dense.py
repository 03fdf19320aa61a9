"""GPU parity of the dense OFT linear path against the fp64 oracle.

Tolerances: outputs and gradients max|a - ref| / max|ref| <= 2e-2 (bf16
matrix-core arithmetic); fp32 R orthogonality <= 1e-3; dequantised weights
bit-exact.
"""
import numpy as np
import pytest

from oft_inputs import CONFIGS, DenseConfig, make_dense
from oracle import codec, dense as odense
from tests.helpers import bf16_to_f64, dev, err, host

pytestmark = pytest.mark.gpu
TOL = 2e-2

SMALL = {
    "tiny_qkv": CONFIGS["tiny_qkv"],
    # several tiles in every dimension, ragged M / N / n-step / K tile
    "fp8_b32_ragged": DenseConfig("fp8_b32_ragged", M=300, K=512, segs=(256, 64, 96), b=32,
                                  x_dtype="bf16", w_fmt="fp8"),
    "int4_g64_ragged_k": DenseConfig("int4_g64_ragged_k", M=520, K=576, segs=(320, 320), b=32,
                                     x_dtype="bf16", w_fmt="int4", g=64),
    "int4_g128_b16": DenseConfig("int4_g128_b16", M=257, K=384, segs=(160, 96), b=16,
                                 x_dtype="bf16", w_fmt="int4", g=128, q_std=0.05),
    "fp8_b16_f32x": DenseConfig("fp8_b16_f32x", M=70, K=128, segs=(48, 16, 32), b=16,
                                x_dtype="f32", w_fmt="fp8"),
    "int4_g32_f32x_b32": DenseConfig("int4_g32_f32x_b32", M=33, K=256, segs=(64, 32), b=32,
                                     x_dtype="f32", w_fmt="int4", g=32),
    "fp8_b16_bf16x": DenseConfig("fp8_b16_bf16x", M=200, K=320, segs=(96, 64, 32), b=16,
                                 x_dtype="bf16", w_fmt="fp8"),
    "int4_g32_bf16x": DenseConfig("int4_g32_bf16x", M=129, K=192, segs=(288,), b=32,
                                  x_dtype="bf16", w_fmt="int4", g=32),
    # wide layers, many tokens: dX through the transposed weight, fp32 dX
    "fp8_f32x_wide": DenseConfig("fp8_f32x_wide", M=150, K=320, segs=(64, 64), b=32,
                                 x_dtype="f32", w_fmt="fp8"),
    "int4_f32x_wide": DenseConfig("int4_f32x_wide", M=140, K=384, segs=(96, 96), b=16,
                                  x_dtype="f32", w_fmt="int4", g=64),
    # fp32 x, INT4, K % 256 == 0: the bf16-x route reads the codes in place,
    # fp32 dX keeps the transposed bf16 copy
    "int4_f32x_k512_wide": DenseConfig("int4_f32x_k512_wide", M=150, K=512, segs=(64, 64), b=32,
                                       x_dtype="f32", w_fmt="int4", g=64),
    "decode_m1": DenseConfig("decode_m1", M=1, K=256, segs=(128, 128), b=32, x_dtype="bf16",
                             w_fmt="int4", g=128),
    # few tokens, wide layer: weight-streaming forward, split-contraction dX
    "decode_split": DenseConfig("decode_split", M=100, K=512, segs=(256, 192), b=32, x_dtype="bf16",
                                w_fmt="int4", g=128),
    "decode_split_fp8_b16": DenseConfig("decode_split_fp8_b16", M=37, K=768, segs=(64, 96), b=16,
                                        x_dtype="bf16", w_fmt="fp8"),
    # few tokens, INT4, K % 256 == 0: weight stream on 256-wide steps (two
    # token tiles, ragged last channel tile; one token tile)
    "decode_int4_g32": DenseConfig("decode_int4_g32", M=48, K=512, segs=(160, 128), b=32, x_dtype="bf16",
                                   w_fmt="int4", g=32),
    "decode_int4_k768_m48": DenseConfig("decode_int4_k768_m48", M=48, K=768, segs=(160, 128), b=32, x_dtype="bf16",
                                        w_fmt="int4", g=32),
    "fp4_decode_k768": DenseConfig("fp4_decode_k768", M=40, K=768, segs=(160, 128), b=32, x_dtype="bf16",
                                   w_fmt="fp4", g=32),
    "decode_int4_g64_b16": DenseConfig("decode_int4_g64_b16", M=20, K=768, segs=(96, 64), b=16,
                                       x_dtype="bf16", w_fmt="int4", g=64),
    # few tokens, 4-bit, more 256-wide steps: odd and even step counts,
    # one and two token tiles, a single row, many channel tiles
    "decode_int4_g128_m64_k1536": DenseConfig("decode_int4_g128_m64_k1536", M=64, K=1536, segs=(320, 256),
                                              b=32, x_dtype="bf16", w_fmt="int4", g=128),
    "decode_int4_g64_b16_m1_k1024": DenseConfig("decode_int4_g64_b16_m1_k1024", M=1, K=1024, segs=(96, 64),
                                                b=16, x_dtype="bf16", w_fmt="int4", g=64, q_std=0.05),
    "decode_fp4_g32_m33_k2048": DenseConfig("decode_fp4_g32_m33_k2048", M=33, K=2048, segs=(128, 64), b=32,
                                            x_dtype="bf16", w_fmt="fp4", g=32),
    # INT4 dX on the split-contraction transposed-code kernel (K % 256 == 0,
    # N % 64 == 0, at most 128 tokens): a full 128-row tile, 3 column tiles
    "decode_int4_q4_m128": DenseConfig("decode_int4_q4_m128", M=128, K=768, segs=(192, 128), b=32,
                                       x_dtype="bf16", w_fmt="int4", g=64),
    "decode_int4_520_blocks_b16": DenseConfig("decode_int4_520_blocks_b16", M=17, K=512, segs=(9600, 7040),
                                              b=16, x_dtype="bf16", w_fmt="int4", g=32, q_std=0.05),
    # FP4 base (OCP MX E2M1 + E8M0 group exponents) through every forward
    # kernel and both dX routes: copy ring with the gemm_nn dX, copy ring
    # with the transposed-weight dX, register prefetch (fp32 x), skinny,
    # 256-wide-step decode, 64-wide-step decode
    "fp4_g32_ragged": DenseConfig("fp4_g32_ragged", M=300, K=512, segs=(256, 64, 96), b=32,
                                  x_dtype="bf16", w_fmt="fp4", g=32),
    "fp4_g64_wide": DenseConfig("fp4_g64_wide", M=200, K=576, segs=(320, 320), b=32,
                                x_dtype="bf16", w_fmt="fp4", g=64),
    "fp4_f32x_b16": DenseConfig("fp4_f32x_b16", M=150, K=384, segs=(96, 96), b=16,
                                x_dtype="f32", w_fmt="fp4", g=64),
    "fp4_skinny_f32x": DenseConfig("fp4_skinny_f32x", M=33, K=256, segs=(64, 32), b=32,
                                   x_dtype="f32", w_fmt="fp4", g=32),
    "fp4_decode_g32": DenseConfig("fp4_decode_g32", M=48, K=512, segs=(160, 128), b=32, x_dtype="bf16",
                                  w_fmt="fp4", g=32),
    "fp4_decode_k576_b16": DenseConfig("fp4_decode_k576_b16", M=20, K=576, segs=(96, 64), b=16,
                                       x_dtype="bf16", w_fmt="fp4", g=64),
    # INT4, bf16 x, many tokens, K % 256 == 0: dX reads the codes through
    # 4-bit transpose loads (ragged row tile, g = 32 and g = 128)
    "int4_q4_dx_g32": DenseConfig("int4_q4_dx_g32", M=300, K=512, segs=(256, 192), b=32, x_dtype="bf16",
                                  w_fmt="int4", g=32),
    "int4_q4_dx_g128_b16": DenseConfig("int4_q4_dx_g128_b16", M=200, K=768, segs=(320, 128), b=16, x_dtype="bf16",
                                       w_fmt="int4", g=128, q_std=0.05),
    # the most segments the ABI takes (8), of unequal sizes, each rotated
    # with its own blocks: copy-ring forward and transposed-weight dX (FP8),
    # and INT4 with b = 16 (gemm_nn dX)
    "fp8_8seg": DenseConfig("fp8_8seg", M=300, K=512, segs=(64, 32, 96, 32, 64, 128, 32, 64), b=32,
                            x_dtype="bf16", w_fmt="fp8"),
    "int4_8seg_b16": DenseConfig("int4_8seg_b16", M=150, K=256, segs=(16, 48, 32, 16, 64, 16, 32, 32), b=16,
                                 x_dtype="bf16", w_fmt="int4", g=32, q_std=0.05),
}


def _wfmt(oft, name):
    return {"int4": oft.OFT_W_INT4, "fp8": oft.OFT_W_FP8_E4M3, "fp4": oft.OFT_W_FP4_E2M1}[name]


def _run_gpu(inp, want_bwd=True):
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = inp["cfg"]
    xdt = oft.OFT_DT_F32 if cfg.x_dtype == "f32" else oft.OFT_DT_BF16
    wf = _wfmt(oft, cfg.w_fmt)
    d = oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, xdt, wf, cfg.g)
    tdt = torch.float32 if cfg.x_dtype == "f32" else torch.int16
    q = dev(inp["p"])
    Rf = torch.empty((cfg.nblk, cfg.b, cfg.b), dtype=torch.float32, device="cuda")
    Rops = torch.empty((cfg.nblk, 2, cfg.b, cfg.b), dtype=torch.int16, device="cuda")
    oft.cayley_build(q, cfg.nblk, cfg.b, Rf, Rops)
    x, wc, ws = dev(inp["x"]), dev(inp["w_codes"]), dev(inp["w_scales"])
    y = torch.empty((cfg.M, cfg.N), dtype=tdt, device="cuda")
    oft.oft_linear_fwd(d, x, wc, ws, Rops, y)
    out = {"Rf": Rf, "Rops": Rops, "y": y}
    if want_bwd:
        dy = dev(inp["dy"])
        dx = torch.empty((cfg.M, cfg.K), dtype=tdt, device="cuda")
        dq = torch.empty((cfg.nblk, cfg.npair), dtype=torch.float32, device="cuda")
        nb = oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD)
        work = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        oft.oft_linear_bwd(d, dy, y, wc, ws, Rf, Rops, dx, dq, work, nb)
        out.update(dx=dx, dq=dq)
    torch.cuda.synchronize()
    return out


def _run_base(inp):
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = inp["cfg"]
    xdt = oft.OFT_DT_F32 if cfg.x_dtype == "f32" else oft.OFT_DT_BF16
    wf = _wfmt(oft, cfg.w_fmt)
    d = oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, xdt, wf, cfg.g)
    tdt = torch.float32 if cfg.x_dtype == "f32" else torch.int16
    y = torch.full((cfg.M, cfg.N), -7, dtype=tdt, device="cuda")
    oft.oft_linear_fwd_base(d, dev(inp["x"]), dev(inp["w_codes"]), dev(inp["w_scales"]), y)
    torch.cuda.synchronize()
    return y


# one case per forward kernel: copy-ring FP8 and INT4 (bf16 x), register-
# prefetch FP8 and INT4 (fp32 x), skinny (fp32 x, few tokens), 4-bit decode
# on 256-wide steps (one and two token tiles, many channel tiles), FP8
# decode
BASE_CASES = ["fp8_b32_ragged", "int4_g64_ragged_k", "fp8_b16_f32x", "int4_f32x_wide", "int4_g32_f32x_b32",
              "decode_int4_g32", "decode_m1", "decode_int4_g64_b16", "decode_split_fp8_b16", "fp4_g64_wide",
              "fp4_decode_g32", "decode_int4_520_blocks_b16"]


@pytest.mark.parametrize("name", BASE_CASES)
def test_base_forward_parity_and_q_zero_identity(name):
    """Reference-policy forward (frozen base, R = I) against the oracle, and
    bit-identical to the adapted forward with Q = 0 (whose R is exactly I);
    with fp32 outputs the adapted path rounds Z to bf16 for the rotation, so
    it equals the base output rounded to bf16."""
    cfg = SMALL[name]
    print(f"[base fwd] {name} M={cfg.M} K={cfg.K} N={cfg.N} {cfg.w_fmt} x {cfg.x_dtype}", flush=True)
    inp = make_dense(cfg, seed=0)
    y_ref = odense.base_forward(odense.x_f64(inp), odense.dequant(inp))
    yb = _run_base(inp)
    e = err(_to64(yb, cfg), y_ref)
    print(f"  err y_base={e:.2e}", flush=True)
    assert e <= TOL
    inp0 = dict(inp)
    inp0["p"] = np.zeros_like(inp["p"])
    y0 = host(_run_gpu(inp0, want_bwd=False)["y"])
    if cfg.x_dtype == "f32":
        rounded = codec.bf16_bits_to_f64(codec.f32_to_bf16_bits(host(yb))).astype(np.float32)
        assert np.array_equal(y0, rounded)
    else:
        assert np.array_equal(y0, host(yb))


def _to64(t, cfg):
    a = host(t)
    return a.astype(np.float64) if cfg.x_dtype == "f32" else bf16_to_f64(a)


@pytest.mark.parametrize("name", list(SMALL))
def test_dense_parity_small(name):
    cfg = SMALL[name]
    print(f"[dense parity] {name} M={cfg.M} K={cfg.K} N={cfg.N} b={cfg.b} {cfg.w_fmt}", flush=True)
    inp = make_dense(cfg, seed=0)
    ref = odense.run(inp)
    out = _run_gpu(inp)
    R = host(out["Rf"]).astype(np.float64)
    orth = np.abs(np.swapaxes(R, 1, 2) @ R - np.eye(cfg.b)).max()
    assert orth <= 1e-3, orth
    assert err(R, ref["R"]) <= 1e-5
    e_y = err(_to64(out["y"], cfg), ref["y"])
    e_dx = err(_to64(out["dx"], cfg), ref["dx"])
    e_dq = err(host(out["dq"]), ref["dp"])
    print(f"  err y={e_y:.2e} dx={e_dx:.2e} dq={e_dq:.2e} orth={orth:.1e}", flush=True)
    assert e_y <= TOL and e_dx <= TOL and e_dq <= TOL


def test_cayley_ops_pack_is_bf16_of_f32():
    import torch

    cfg = SMALL["fp8_b32_ragged"]
    out = _run_gpu(make_dense(cfg, seed=1), want_bwd=False)
    R = host(out["Rf"])
    ops = host(out["Rops"], np.uint16)
    want = codec.f32_to_bf16_bits(R)
    assert np.array_equal(ops[:, 0], want)
    assert np.array_equal(ops[:, 1], np.swapaxes(want, 1, 2))


@pytest.mark.parametrize("fmt,g", [("int4", 32), ("int4", 64), ("int4", 128), ("fp8", 0), ("fp4", 32),
                                   ("fp4", 128)])
def test_dequant_bit_exact(fmt, g):
    import torch
    import orthogonal_fine_tuning_amd as oft

    rows, cols = 96, 512
    cfg = DenseConfig("dq", M=1, K=cols, segs=(rows,), b=32, x_dtype="bf16", w_fmt=fmt, g=g)
    inp = make_dense(cfg, seed=3, with_dy=False)
    if fmt == "fp8":  # every e4m3fn code except NaN, in every row
        codes = np.tile(np.arange(256, dtype=np.uint8), (rows, cols // 256))
        codes[(codes & 0x7F) == 0x7F] = 0
        inp["w_codes"] = codes
        ref = codec.f32_to_bf16_bits(odense.dequant_fp8_codes(codes).astype(np.float32))
    elif fmt == "fp4":  # every exponent code 0 .. 254, the high byte of the slot set (ignored)
        ns = rows * cols // g
        inp["w_scales"] = ((np.arange(ns) % 255) | 0x5A00).astype(np.uint16).reshape(rows, cols // g)
        with np.errstate(over="ignore"):
            ref = codec.f32_to_bf16_bits(odense.dequant_fp4(inp["w_codes"], inp["w_scales"], g)
                                         .astype(np.float32))
    else:
        ref = codec.f32_to_bf16_bits(odense.dequant_int4(inp["w_codes"], inp["w_scales"], g)
                                     .astype(np.float32))
    out = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
    wf = _wfmt(oft, fmt)
    oft.oft_dequant(wf, rows, cols, g, dev(inp["w_codes"]), dev(inp["w_scales"]), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out, np.uint16), ref)


def test_q_zero_gives_plain_dequant_gemm():
    """Q = 0: R = I exactly, so y equals the un-rotated dequant GEMM (to bf16)."""
    cfg = SMALL["int4_g64_ragged_k"]
    inp = make_dense(cfg, seed=2)
    inp["p"] = np.zeros_like(inp["p"])
    out = _run_gpu(inp)
    R = host(out["Rf"])
    assert np.array_equal(R, np.broadcast_to(np.eye(cfg.b, dtype=np.float32), R.shape))
    W = odense.dequant(inp)
    ref = odense.x_f64(inp) @ W.T
    assert err(_to64(out["y"], cfg), ref) <= TOL
    # dq at Q = 0 follows the closed form 2 (G_il - G_li); compared to the oracle
    assert err(host(out["dq"]), odense.run(inp)["dp"]) <= TOL


def test_m_zero_is_noop_and_dq_zero():
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = SMALL["fp8_b32_ragged"].with_(M=0)
    d = oft.linear_desc(0, cfg.K, cfg.segs, cfg.b, oft.OFT_DT_BF16, oft.OFT_W_FP8_E4M3, 0)
    inp = make_dense(cfg.with_(M=1), seed=0)
    q = dev(inp["p"])
    Rf = torch.empty((cfg.nblk, 32, 32), dtype=torch.float32, device="cuda")
    Rops = torch.empty((cfg.nblk, 2, 32, 32), dtype=torch.int16, device="cuda")
    oft.cayley_build(q, cfg.nblk, 32, Rf, Rops)
    dq = torch.full((cfg.nblk, cfg.npair), 7.0, dtype=torch.float32, device="cuda")
    nb = oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD)
    work = torch.empty(nb, dtype=torch.uint8, device="cuda")
    wc, ws = dev(inp["w_codes"]), dev(inp["w_scales"])
    oft.oft_linear_fwd(d, None, wc, ws, Rops, None)
    oft.oft_linear_bwd(d, None, None, wc, ws, Rf, Rops, None, dq, work, nb)
    torch.cuda.synchronize()
    assert np.all(host(dq) == 0.0)


def test_deterministic_bitwise():
    cfg = SMALL["fp8_b32_ragged"]
    inp = make_dense(cfg, seed=4)
    a = _run_gpu(inp)
    b = _run_gpu(inp)
    for k in ("y", "dx", "dq"):
        assert np.array_equal(host(a[k]), host(b[k])), k


# the QKV layer at 3072 tokens: the forward picks 192-token tiles (128-wide
# K steps at that tile size) and dX 128-token tiles
# and the gate/up workloads on an FP4 base, as `bench.py --w-fmt fp4` times them
FULL_EXTRA = {"qkv_3072": CONFIGS["qkv_4b"].with_(name="qkv_3072", M=3072),
              "gateup_4b_train_fp4": CONFIGS["gateup_4b_train"].with_(name="gateup_4b_train_fp4", w_fmt="fp4"),
              "gateup_4b_decode_fp4": CONFIGS["gateup_4b_decode"].with_(name="gateup_4b_decode_fp4", w_fmt="fp4")}


@pytest.mark.parametrize("name", ["qkv_4b", "gateup_4b_train", "gateup_4b_decode", "qkv_3072", "gateup_4b_train_fp4",
                                  "gateup_4b_decode_fp4"])
def test_dense_full_size(name):
    """Full workload shapes in the launch configuration the benchmark times:
    every element of y and dX and every block of dQ against the oracle."""
    cfg = FULL_EXTRA[name] if name in FULL_EXTRA else CONFIGS[name]
    print(f"[dense full size] {name}: M={cfg.M} K={cfg.K} N={cfg.N} {cfg.w_fmt}", flush=True)
    inp = make_dense(cfg, seed=0)
    out = _run_gpu(inp)
    gy, gdx, gdq = _to64(out["y"], cfg), _to64(out["dx"], cfg), host(out["dq"])
    R32 = host(out["Rf"]).astype(np.float64)
    del out
    print(f"[dense full size] {name}: oracle", flush=True)
    ref = odense.run(inp)
    e_y = err(gy, ref["y"])
    e_dx = err(gdx, ref["dx"])
    e_dq = err(gdq, ref["dp"])
    orth = np.abs(np.swapaxes(R32, 1, 2) @ R32 - np.eye(cfg.b)).max()
    # per token tile of 128 rows and per adapter block, the worst error, so
    # that one tile computed wrongly cannot hide in the normwise figure
    den_y = np.abs(ref["y"]).max()
    tile_y = max(np.abs(gy[m:m + 128] - ref["y"][m:m + 128]).max() for m in range(0, cfg.M, 128)) / den_y
    print(f"  err y={e_y:.2e} dx={e_dx:.2e} dq={e_dq:.2e} worst y tile={tile_y:.2e} orth={orth:.1e}", flush=True)
    assert max(e_y, e_dx, e_dq) <= TOL and orth <= 1e-3
    for j in range(cfg.nblk):
        assert err(gdq[j], ref["dp"][j]) <= 5 * TOL, j  # blockwise: a wrong block fails even if small


@pytest.mark.parametrize("b,nblk", [(32, 3001), (16, 3001), (32, 37), (16, 37), (16, 1), (32, 1)])
def test_cayley_many_blocks(b, nblk):
    """Many blocks (one lane per row), and few (two lanes per row: the build
    of a dense layer), the last wave holding fewer blocks than it can."""
    import torch
    import orthogonal_fine_tuning_amd as oft
    from oft_inputs import to_bf16_bits

    rng = np.random.default_rng(b)
    p = to_bf16_bits(rng.normal(0.0, 0.3, size=(nblk, b * (b - 1) // 2)).astype(np.float32))
    Rf = torch.empty((nblk, b, b), dtype=torch.float32, device="cuda")
    Rops = torch.empty((nblk, 2, b, b), dtype=torch.int16, device="cuda")
    oft.cayley_build(dev(p), nblk, b, Rf, Rops)
    torch.cuda.synchronize()
    R = host(Rf).astype(np.float64)
    ref = odense.cayley(p, b)
    assert err(R, ref) <= 1e-5
    assert np.abs(np.swapaxes(R, 1, 2) @ R - np.eye(b)).max() <= 1e-3
    ops = host(Rops, np.uint16)
    assert np.array_equal(ops[:, 0], codec.f32_to_bf16_bits(host(Rf)))
    assert np.array_equal(ops[:, 1], np.swapaxes(ops[:, 0], 1, 2))
