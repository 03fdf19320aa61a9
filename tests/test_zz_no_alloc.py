"""oft_linear_bwd_noalloc (the dense backward on the library's fixed scratch
array, for callers that cannot allocate) against oft_linear_bwd with a
caller workspace: bit for bit (same kernels, same plan), on two calls in a
row, the second with a smaller layer, and against the oracle."""
import numpy as np
import pytest

from oft_inputs import CONFIGS, DenseConfig, make_dense
from oracle import dense as odense
from tests.helpers import bf16_to_f64, dev, err, host

pytestmark = pytest.mark.gpu


def _setup(cfg, seed):
    import torch
    import orthogonal_fine_tuning_amd as oft

    inp = make_dense(cfg, seed=seed)
    wf = {"int4": oft.OFT_W_INT4, "fp8": oft.OFT_W_FP8_E4M3, "fp4": oft.OFT_W_FP4_E2M1}[cfg.w_fmt]
    xdt = oft.OFT_DT_F32 if cfg.x_dtype == "f32" else oft.OFT_DT_BF16
    tdt = torch.float32 if cfg.x_dtype == "f32" else torch.int16
    d = oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, xdt, wf, cfg.g)
    t = {"d": d, "inp": inp, "tdt": tdt}
    t["Rf"] = torch.empty((cfg.nblk, cfg.b, cfg.b), dtype=torch.float32, device="cuda")
    t["Rops"] = torch.empty((cfg.nblk, 2, cfg.b, cfg.b), dtype=torch.int16, device="cuda")
    oft.cayley_build(dev(inp["p"]), cfg.nblk, cfg.b, t["Rf"], t["Rops"])
    for k in ("x", "w_codes", "w_scales", "dy"):
        t[k] = dev(inp[k])
    t["y"] = torch.empty((cfg.M, cfg.N), dtype=tdt, device="cuda")
    oft.oft_linear_fwd(d, t["x"], t["w_codes"], t["w_scales"], t["Rops"], t["y"])
    return t


def _bwd(cfg, t, noalloc):
    import torch
    import orthogonal_fine_tuning_amd as oft

    dx = torch.full((cfg.M, cfg.K), 3, dtype=t["tdt"], device="cuda")
    dq = torch.full((cfg.nblk, cfg.npair), 5.0, dtype=torch.float32, device="cuda")
    if noalloc:
        oft.oft_linear_bwd_noalloc(t["d"], t["dy"], t["y"], t["w_codes"], t["w_scales"], t["Rf"], t["Rops"], dx, dq)
    else:
        nb = oft.oft_linear_workspace_bytes(t["d"], oft.OFT_PASS_BWD)
        work = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        oft.oft_linear_bwd(t["d"], t["dy"], t["y"], t["w_codes"], t["w_scales"], t["Rf"], t["Rops"], dx, dq, work, nb)
    torch.cuda.synchronize()
    return host(dx), host(dq)


# a large layer first (the whole 4096-token QKV layer: 75 MiB of scratch,
# transposed-weight dX), then smaller ones reusing the array's stale contents
CASES = [CONFIGS["qkv_4b"],
         DenseConfig("small_int4", M=300, K=512, segs=(256, 64, 96), b=32, x_dtype="bf16", w_fmt="int4", g=64),
         CONFIGS["gateup_4b_decode"]]


def test_noalloc_matches_workspace_call_twice_in_a_row():
    for i, cfg in enumerate(CASES):
        print(f"[noalloc] call {i}: {cfg.name} M={cfg.M} K={cfg.K} N={cfg.N} {cfg.w_fmt}", flush=True)
        t = _setup(cfg, seed=i)
        dx_a, dq_a = _bwd(cfg, t, noalloc=True)
        dx_w, dq_w = _bwd(cfg, t, noalloc=False)
        assert np.array_equal(dx_a, dx_w) and np.array_equal(dq_a, dq_w), cfg.name
        if cfg.M <= 512:
            ref = odense.run(t["inp"])
            e_dx = err(bf16_to_f64(dx_a), ref["dx"])
            e_dq = err(dq_a, ref["dp"])
            print(f"  err dx={e_dx:.2e} dq={e_dq:.2e}", flush=True)
            assert e_dx <= 2e-2 and e_dq <= 2e-2


def test_noalloc_rejects_layers_beyond_the_scratch():
    import orthogonal_fine_tuning_amd as oft
    from orthogonal_fine_tuning_amd import _lib

    cfg = CONFIGS["gateup_4b_train"]
    d = oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, oft.OFT_DT_BF16, oft.OFT_W_INT4, cfg.g)
    assert oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD) > _lib.OFT_NOALLOC_SCRATCH_BYTES
    with pytest.raises(oft.OftError) as ei:
        t = _setup(CONFIGS["gateup_4b_decode"], seed=9)  # any valid device pointers
        oft.oft_linear_bwd_noalloc(d, t["dy"], t["y"], t["w_codes"], t["w_scales"], t["Rf"], t["Rops"], t["y"],
                                   t["Rf"])
    assert ei.value.status == _lib.OFT_EWORKSPACE
