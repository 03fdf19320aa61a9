"""GPU parity of the MoE path (routing, grouped fwd, bwd) against the oracle.

Routing tables must match bit for bit; outputs and gradients to
max|a - ref| / max|ref| <= 2e-2; combine weights to 1e-5 relative.
Full-size configurations are checked on sampled tokens (y, dX, dw) and
sampled experts (dQ), which the oracle computes one by one.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oft_inputs import CONFIGS, MoEConfig, make_moe, make_moe_logits
from oracle import codec, moe as omoe
from tests.helpers import bf16_to_f64, dev, err, host

pytestmark = pytest.mark.gpu
TOL = 2e-2

SMALL = {
    # ragged against 64-token count tiles and 128-row GEMM tiles
    "moe_small_b32": MoEConfig("moe_small_b32", T=300, E=16, k=4, H=256, I=128, g=32, chunk=3, b=32,
                               q_std=0.05),
    "moe_small_b16_g64": MoEConfig("moe_small_b16_g64", T=200, E=12, k=3, H=192, I=192, g=64, chunk=5,
                                   b=16, q_std=0.05),
    "moe_small_g128": MoEConfig("moe_small_g128", T=77, E=8, k=2, H=384, I=256, g=128, chunk=2, b=32,
                                bias_std=0.5),
    # at least 64 rows per expert on average (the copy-ring grouped GEMMs);
    # I = 192 leaves a half-filled 128-channel gate/up tile
    "moe_dense_b16_g64": MoEConfig("moe_dense_b16_g64", T=256, E=4, k=2, H=192, I=192, g=64, chunk=2,
                                   b=16, q_std=0.05),
    "moe_dense_g128": MoEConfig("moe_dense_g128", T=300, E=4, k=2, H=384, I=256, g=128, chunk=3, b=32,
                                bias_std=0.5),
    # at most 8 rows per expert on average (16-row weight-streaming tiles);
    # the hot expert spans several of them.  H, I multiples of 256 take the
    # 256-wide-step kernels (and I = 128 the 64-wide-step one for the down
    # projection)
    "moe_decode16_b32": MoEConfig("moe_decode16_b32", T=40, E=32, k=4, H=512, I=256, g=32, chunk=3, b=32,
                                  q_std=0.05),
    "moe_decode16_b16_g64": MoEConfig("moe_decode16_b16_g64", T=24, E=16, k=3, H=256, I=256, g=64, chunk=5,
                                      b=16, q_std=0.05),
    "moe_decode16_i128": MoEConfig("moe_decode16_i128", T=40, E=32, k=4, H=256, I=128, g=32, chunk=3, b=32,
                                   q_std=0.05),
    "moe_decode16_g128": MoEConfig("moe_decode16_g128", T=30, E=32, k=2, H=256, I=256, g=128, chunk=4, b=32,
                                   q_std=0.05, bias_std=0.5),
    # 9 to 63 rows per expert on average: 64-row weight-streaming tiles
    "moe_dec64_g128": MoEConfig("moe_dec64_g128", T=100, E=16, k=4, H=256, I=256, g=128, chunk=4, b=32,
                                q_std=0.05),
    # FP4 experts (OCP MX E2M1 + E8M0 group exponents) through each grouped
    # kernel family: copy ring, 16- and 64-row weight streams on 256-wide
    # steps, and on 64-wide steps (H % 256 != 0)
    "moe_small_fp4": MoEConfig("moe_small_fp4", T=300, E=16, k=4, H=256, I=128, g=32, chunk=3, b=32,
                               q_std=0.05, w_fmt="fp4"),
    "moe_dense_fp4_b16_g64": MoEConfig("moe_dense_fp4_b16_g64", T=256, E=4, k=2, H=192, I=192, g=64, chunk=2,
                                       b=16, q_std=0.05, w_fmt="fp4"),
    "moe_decode16_fp4": MoEConfig("moe_decode16_fp4", T=40, E=32, k=4, H=512, I=256, g=32, chunk=3, b=32,
                                  q_std=0.05, w_fmt="fp4"),
    "moe_dec64_fp4_g128": MoEConfig("moe_dec64_fp4_g128", T=100, E=16, k=4, H=256, I=256, g=128, chunk=4,
                                    b=32, q_std=0.05, w_fmt="fp4"),
    "moe_decode_fp4_h192": MoEConfig("moe_decode_fp4_h192", T=24, E=16, k=3, H=192, I=192, g=64, chunk=5,
                                     b=16, q_std=0.05, w_fmt="fp4"),
}


def _wfmt(oft, name):
    return {"int4": oft.OFT_W_INT4, "fp4": oft.OFT_W_FP4_E2M1}[name]


def _routing_tensors(T, E, k):
    import torch

    P = T * k
    z = lambda *s, dt=torch.int32: torch.full(s, -7, dtype=dt, device="cuda")  # noqa: E731
    return dict(topk_idx=z(max(T, 1), k), topk_w=z(max(T, 1), k, dt=torch.float32), counts=z(E),
                offsets=z(E + 1), perm=z(max(P, 1)), inv_perm=z(max(P, 1)), active=z(E), n_active=z(4),
                chunk_of_expert=z(E))


def _run_route(cfg, logits, renorm=0):
    import torch
    import orthogonal_fine_tuning_amd as oft

    d = oft.moe_desc(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.g, cfg.b, cfg.chunk, renorm)
    rtt = _routing_tensors(cfg.T, cfg.E, cfg.k)
    rt = oft.moe_routing(**rtt)
    nb = oft.oft_moe_workspace_bytes(d, oft.OFT_PASS_FWD)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    oft.oft_moe_route(d, dev(logits), rt, ws, nb)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in rtt.items()}


def _check_routing(cfg, logits, got, renorm=False):
    idx, w = omoe.route(logits, cfg.k, renorm=renorm)
    g = omoe.group(idx, cfg.E, cfg.chunk)
    T, E, k = cfg.T, cfg.E, cfg.k
    assert np.array_equal(got["topk_idx"][:T], idx)
    assert np.abs(got["topk_w"][:T] - w).max() <= 1e-5 * max(1e-30, np.abs(w).max())
    assert np.array_equal(got["counts"], g["counts"])
    assert np.array_equal(got["offsets"], g["offsets"])
    assert np.array_equal(got["perm"][:T * k], g["perm"])
    assert np.array_equal(got["inv_perm"][:T * k], g["inv_perm"])
    assert got["n_active"][0] == g["n_active"]
    assert np.array_equal(got["active"][:g["n_active"]], g["active"])
    assert np.all(got["active"][g["n_active"]:] == -1)
    assert np.array_equal(got["chunk_of_expert"], g["chunk_of_expert"])


@pytest.mark.parametrize("name", ["moe_30b_a3b", "moe_1t_train", "moe_1t_decode"])
def test_routing_bit_exact_config_logits(name):
    cfg = CONFIGS[name]
    print(f"[moe routing] {name} T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    logits = make_moe_logits(cfg, seed=0)
    _check_routing(cfg, logits, _run_route(cfg, logits))


# router-only shapes for the lane-group widths the small configurations miss
# (33 .. 64 experts: 16 lanes per token; 129 .. 256: 32; 385 .. 512 and
# 513 .. 1024: 64 with 8 and 16 logits per lane)
ROUTER = {
    "router_e60": MoEConfig("router_e60", T=45, E=60, k=5, H=64, I=64, g=32, chunk=4, b=32),
    "router_e200": MoEConfig("router_e200", T=77, E=200, k=6, H=64, I=64, g=32, chunk=4, b=32, bias_std=0.5),
    "router_e500": MoEConfig("router_e500", T=50, E=500, k=16, H=64, I=64, g=32, chunk=4, b=32),
    "router_e1000": MoEConfig("router_e1000", T=33, E=1000, k=16, H=64, I=64, g=32, chunk=4, b=32, bias_std=0.5),
}


@pytest.mark.parametrize("name,renorm", [("moe_small_b32", 0), ("moe_small_g128", 1), ("moe_decode16_b32", 1),
                                         ("moe_30b_a3b", 0), ("moe_1t_decode", 1), ("moe_1t_train", 0),
                                         ("router_e60", 1), ("router_e200", 0), ("router_e200", 1),
                                         ("router_e500", 0), ("router_e1000", 1)])
def test_router_backward(name, renorm):
    """d_logits through the softmax top-k, the selection from the GPU routing
    (bit-exact against the oracle's) and a seeded dw, against the oracle."""
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = SMALL.get(name) or ROUTER.get(name) or CONFIGS[name]
    print(f"[router bwd] {name} T={cfg.T} E={cfg.E} k={cfg.k} renorm={renorm}", flush=True)
    logits = make_moe_logits(cfg, seed=0)
    got = _run_route(cfg, logits, renorm=renorm)
    _check_routing(cfg, logits, got, renorm=bool(renorm))  # the top-k of every lane-group shape, bit-exact
    idx = got["topk_idx"][:cfg.T]
    dw = np.random.default_rng(7).standard_normal((cfg.T, cfg.k)).astype(np.float32)
    d = oft.moe_desc(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.g, cfg.b, cfg.chunk, renorm)
    dl = torch.full((cfg.T, cfg.E), -7.0, dtype=torch.float32, device="cuda")
    oft.oft_moe_router_bwd(d, dev(logits), dev(idx), dev(dw), dl)
    torch.cuda.synchronize()
    ref = omoe.router_backward(logits, idx, dw, renorm=bool(renorm))
    e = err(host(dl), ref)
    print(f"  err d_logits={e:.2e}", flush=True)
    assert e <= 1e-5
    if renorm:  # only the selected experts get a gradient
        mask = np.ones((cfg.T, cfg.E), dtype=bool)
        mask[np.arange(cfg.T)[:, None], idx] = False
        assert np.all(host(dl)[mask] == 0.0)


def test_routing_ties_and_renorm():
    cfg = MoEConfig("ties", T=1000, E=96, k=8, H=64, I=64, g=32, chunk=7, b=32)
    rng = np.random.default_rng(9)
    logits = rng.integers(-3, 4, size=(cfg.T, cfg.E)).astype(np.float32)  # massive ties
    logits[5, :] = 0.0
    logits[:, 40] -= 100.0  # expert 40 never chosen
    got = _run_route(cfg, logits)
    _check_routing(cfg, logits, got)
    assert got["topk_idx"][5].tolist() == list(range(8))
    got = _run_route(cfg, logits, renorm=1)
    _check_routing(cfg, logits, got, renorm=True)


def _bf16_weights(inp):
    """The experts' weights dequantised to bf16 on the GPU (oft_dequant)."""
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = inp["cfg"]
    E, H, I, g = cfg.E, cfg.H, cfg.I, cfg.g
    wgu = torch.empty((E, 2 * I, H), dtype=torch.int16, device="cuda")
    wd = torch.empty((E, H, I), dtype=torch.int16, device="cuda")
    wf = _wfmt(oft, cfg.w_fmt)
    oft.oft_dequant(wf, E * 2 * I, H, g, dev(inp["wgu_codes"]), dev(inp["wgu_scales"]), wgu)
    oft.oft_dequant(wf, E * H, I, g, dev(inp["wd_codes"]), dev(inp["wd_scales"]), wd)
    return {"wgu_codes": wgu, "wgu_scales": None, "wd_codes": wd, "wd_scales": None}


def _run_moe(inp, want_bwd=True, bf16_weights=False):
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = inp["cfg"]
    T, E, k, H, I, b = cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.b
    P = T * k
    w_fmt = oft.OFT_W_BF16 if bf16_weights else _wfmt(oft, cfg.w_fmt)
    d = oft.moe_desc(T, E, k, H, I, cfg.g, b, cfg.chunk, 0, w_fmt=w_fmt)
    rtt = _routing_tensors(T, E, k)
    rt = oft.moe_routing(**rtt)
    nblk = E * cfg.nblk_e
    Rf = torch.empty((E, cfg.nblk_e, b, b), dtype=torch.float32, device="cuda")
    Rops = torch.empty((E, cfg.nblk_e, 2, b, b), dtype=torch.int16, device="cuda")
    oft.cayley_build(dev(inp["p"]), nblk, b, Rf, Rops)
    if bf16_weights:
        W = _bf16_weights(inp)
    else:
        W = {n: dev(inp[n]) for n in ("wgu_codes", "wgu_scales", "wd_codes", "wd_scales")}
    hs = torch.empty((max(P, 1), 2 * I), dtype=torch.int16, device="cuda")
    y = torch.empty((max(T, 1), H), dtype=torch.int16, device="cuda")
    nbf = oft.oft_moe_workspace_bytes(d, oft.OFT_PASS_FWD)
    wsf = torch.empty(nbf, dtype=torch.uint8, device="cuda")
    x = dev(inp["x"]) if T > 0 else torch.empty((1, H), dtype=torch.int16, device="cuda")
    lg = dev(inp["logits"]) if T > 0 else torch.empty((1, E), dtype=torch.float32, device="cuda")
    oft.oft_moe_grouped_fwd(d, x, lg, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"], Rops,
                            rt, hs, y, wsf, nbf)
    out = {"rt": rtt, "hs": hs, "y": y}
    if want_bwd:
        dy = dev(inp["dy"]) if T > 0 else torch.empty((1, H), dtype=torch.int16, device="cuda")
        dx = torch.empty((max(T, 1), H), dtype=torch.int16, device="cuda")
        dq = torch.full((E, cfg.nblk_e, cfg.npair), 3.0, dtype=torch.float32, device="cuda")
        dw = torch.empty((max(T, 1), k), dtype=torch.float32, device="cuda")
        nbb = oft.oft_moe_workspace_bytes(d, oft.OFT_PASS_BWD)
        wsb = torch.empty(nbb, dtype=torch.uint8, device="cuda")
        oft.oft_moe_grouped_bwd(d, dy, rt, hs, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"],
                                Rf, Rops, dx, dq, dw, wsb, nbb)
        out.update(dx=dx, dq=dq, dw=dw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(SMALL))
def test_moe_parity_small(name):
    cfg = SMALL[name]
    print(f"[moe parity] {name}", flush=True)
    inp = make_moe(cfg, seed=0)
    # one inactive expert and one hot expert spanning several 128-row tiles
    inp["logits"] = inp["logits"].copy()
    inp["logits"][:, 1] -= 100.0
    inp["logits"][:, 2] += 3.0
    y_ref, H_ref, rt = omoe.forward(inp)
    dX_ref, dp_ref, dw_ref = omoe.backward(inp, rt)
    out = _run_moe(inp)
    got_rt = {k: host(v) for k, v in out["rt"].items()}
    _check_routing(cfg, inp["logits"], got_rt)
    assert rt["counts"][1] == 0
    if cfg.T > 128:  # the hot expert spans several 128-row tiles
        assert rt["counts"][2] > 128
    P = cfg.T * cfg.k
    e_y = err(bf16_to_f64(host(out["y"])), y_ref)
    e_h = err(bf16_to_f64(host(out["hs"])[:P]), H_ref)
    e_dx = err(bf16_to_f64(host(out["dx"])), dX_ref)
    e_dq = err(host(out["dq"]), dp_ref)
    e_dw = err(host(out["dw"]), dw_ref)
    print(f"  err y={e_y:.2e} h={e_h:.2e} dx={e_dx:.2e} dq={e_dq:.2e} dw={e_dw:.2e}", flush=True)
    assert max(e_y, e_h, e_dx, e_dq, e_dw) <= TOL
    assert np.all(host(out["dq"])[1] == 0.0)  # inactive expert


@pytest.mark.parametrize("name", list(SMALL))
def test_moe_bf16_weights_small(name):
    """Dequantised bf16 weights (the dense reference the grouped dequant GEMMs
    are measured against) through the same entry points: the oracle's result;
    where both formats run the 128-row copy-ring kernels (at least 64 rows per
    expert on average) the contraction order is the same, so every output
    equals the INT4 run's bit for bit."""
    cfg = SMALL[name]
    print(f"[moe bf16 weights] {name}", flush=True)
    inp = make_moe(cfg, seed=3)
    y_ref, H_ref, rt = omoe.forward(inp)
    dX_ref, dp_ref, dw_ref = omoe.backward(inp, rt)
    out = _run_moe(inp, bf16_weights=True)
    P = cfg.T * cfg.k
    e_y = err(bf16_to_f64(host(out["y"])), y_ref)
    e_h = err(bf16_to_f64(host(out["hs"])[:P]), H_ref)
    e_dx = err(bf16_to_f64(host(out["dx"])), dX_ref)
    e_dq = err(host(out["dq"]), dp_ref)
    e_dw = err(host(out["dw"]), dw_ref)
    print(f"  err y={e_y:.2e} h={e_h:.2e} dx={e_dx:.2e} dq={e_dq:.2e} dw={e_dw:.2e}", flush=True)
    assert max(e_y, e_h, e_dx, e_dq, e_dw) <= TOL
    if P >= 64 * cfg.E:
        ref = _run_moe(inp)
        for key in ("y", "hs", "dx", "dq", "dw"):
            assert np.array_equal(host(out[key]), host(ref[key])), key


def test_moe_deterministic():
    cfg = SMALL["moe_small_b32"]
    inp = make_moe(cfg, seed=5)
    a, b = _run_moe(inp), _run_moe(inp)
    for key in ("y", "hs", "dx", "dq", "dw"):
        assert np.array_equal(host(a[key]), host(b[key])), key


def test_moe_zero_tokens():
    cfg = SMALL["moe_small_b32"].with_(T=0)
    inp = make_moe(cfg.with_(T=1), seed=1)
    inp["cfg"] = cfg
    out = _run_moe(inp)
    assert np.all(host(out["dq"]) == 0.0)
    assert np.all(host(out["rt"]["counts"]) == 0)
    assert host(out["rt"]["n_active"])[0] == 0


# ------------------------------------------------------------ full size, sampled
def _sampled_reference(inp, tokens, experts, threads=16):
    cfg = inp["cfg"]
    k = cfg.k
    idx, w = omoe.route(inp["logits"], k)
    rt = omoe.group(idx, cfg.E, cfg.chunk)
    X = codec.bf16_bits_to_f64(inp["x"])
    dy = codec.bf16_bits_to_f64(inp["dy"])
    wflat = w.reshape(-1)
    need = sorted(set(int(idx[t, j]) for t in tokens for j in range(k)) | set(experts))

    def one(e):
        pairs_all = rt["perm"][rt["offsets"][e]:rt["offsets"][e + 1]]
        sel = [p for p in pairs_all if p // k in set(tokens)]
        Wgu, Wd, R = omoe.expert_weights(inp, e)
        res = {}
        if sel:
            sel = np.asarray(sel)
            _, _, _, O = omoe.expert_forward(X[sel // k], Wgu, Wd, R, cfg.I)
            dwe, _, dXp = omoe.expert_backward(inp, e, sel, X, dy, wflat)
            res["tok"] = (sel, O, dwe, dXp)
        if e in experts:
            res["dp"] = omoe.expert_backward(inp, e, pairs_all, X, dy, wflat)[1] if len(pairs_all) else \
                np.zeros((cfg.nblk_e, cfg.npair))
        return e, res

    with ThreadPoolExecutor(threads) as ex:
        results = dict(ex.map(one, need))
    y = {t: np.zeros(cfg.H) for t in tokens}
    dx = {t: np.zeros(cfg.H) for t in tokens}
    dw = {}
    for e, res in results.items():
        if "tok" in res:
            sel, O, dwe, dXp = res["tok"]
            for r, p in enumerate(sel):
                t = int(p // k)
                y[t] += wflat[p] * O[r]
                dx[t] += dXp[r]
                dw[int(p)] = dwe[r]
    dp = {e: results[e]["dp"] for e in experts}
    return rt, y, dx, dw, dp


# the MoE workloads on FP4 experts, as `bench.py --w-fmt fp4` times them
MOE_FULL_FP4 = {n + "_fp4": CONFIGS[n].with_(name=n + "_fp4", w_fmt="fp4") for n in ("moe_30b_a3b", "moe_1t_decode")}


@pytest.mark.parametrize("name", ["moe_30b_a3b", "moe_1t_train", "moe_1t_decode", "moe_30b_a3b_fp4",
                                  "moe_1t_decode_fp4"])
def test_moe_full_size_sampled(name):
    cfg = MOE_FULL_FP4.get(name) or CONFIGS[name]
    print(f"[moe full size] {name}: generating inputs", flush=True)
    inp = make_moe(cfg, seed=0)
    print(f"[moe full size] {name}: GPU fwd+bwd", flush=True)
    out = _run_moe(inp)
    counts = host(out["rt"]["counts"])
    order = np.argsort(-counts, kind="stable")
    experts = [int(order[0]), int(order[len(order) // 2])]
    inactive = np.nonzero(counts == 0)[0]
    tokens = [0, cfg.T // 3, cfg.T - 1]
    print(f"[moe full size] {name}: oracle on tokens {tokens}, experts {experts}", flush=True)
    rt, y, dx, dw, dp = _sampled_reference(inp, tokens, experts)
    assert np.array_equal(counts, rt["counts"])
    gy = bf16_to_f64(host(out["y"]))
    gdx = bf16_to_f64(host(out["dx"]))
    gdw = host(out["dw"]).reshape(-1)
    gdq = host(out["dq"])
    e_y = err(np.stack([gy[t] for t in tokens]), np.stack([y[t] for t in tokens]))
    e_dx = err(np.stack([gdx[t] for t in tokens]), np.stack([dx[t] for t in tokens]))
    ps = sorted(dw)
    e_dw = err(gdw[ps], np.array([dw[p] for p in ps]))
    e_dq = max(err(gdq[e], dp[e]) for e in experts)
    print(f"  err y={e_y:.2e} dx={e_dx:.2e} dw={e_dw:.2e} dq={e_dq:.2e} inactive={len(inactive)}", flush=True)
    assert max(e_y, e_dx, e_dw, e_dq) <= TOL
    for e in inactive[:8]:
        assert np.all(gdq[e] == 0.0)
