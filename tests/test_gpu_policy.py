"""The per-token log-probability difference of two policies (the KL
estimate between the adapted layer and the frozen base alone) against the
oracle, and end to end on a dense layer's outputs used as logits."""
import numpy as np
import pytest

from oft_inputs import DenseConfig, make_dense
from oracle import dense as odense, policy
from tests.helpers import bf16_to_f64, dev, err, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,V,scale,shift", [(1, 1, 1.0, 0.0), (5, 7, 2.0, 0.0), (37, 1000, 3.0, 0.0),
                                             (8, 151936, 4.0, 0.0), (16, 4097, 1.0, 800.0), (3, 256, 30.0, -50.0)])
def test_logprob_diff_against_oracle(T, V, scale, shift):
    import torch
    import orthogonal_fine_tuning_amd as oft

    rng = np.random.default_rng(T * 1000 + V)
    a = (rng.normal(0, scale, (T, V)) + shift).astype(np.float32)
    r = rng.normal(0, scale, (T, V)).astype(np.float32)
    lab = rng.integers(0, V, T).astype(np.int32)
    out = torch.full((T,), 9.0, dtype=torch.float32, device="cuda")
    oft.oft_logprob_diff(dev(a), dev(r), dev(lab), out)
    torch.cuda.synchronize()
    ref = policy.logprob_diff(a, r, lab)
    got = host(out).astype(np.float64)
    e = np.abs(got - ref).max()
    print(f"[logprob diff] T={T} V={V}: max abs err {e:.2e}", flush=True)
    assert e <= 1e-4 * max(1.0, np.abs(ref).max())
    same = torch.empty_like(out)
    oft.oft_logprob_diff(dev(a), dev(a), dev(lab), same)
    torch.cuda.synchronize()
    assert np.all(host(same) == 0.0)  # the same policy twice: exactly zero


def test_logprob_diff_bad_label_is_nan():
    import torch
    import orthogonal_fine_tuning_amd as oft

    a = np.zeros((3, 10), dtype=np.float32)
    lab = np.array([2, -1, 10], dtype=np.int32)
    out = torch.zeros(3, dtype=torch.float32, device="cuda")
    oft.oft_logprob_diff(dev(a), dev(a), dev(lab), out)
    torch.cuda.synchronize()
    o = host(out)
    assert o[0] == 0.0 and np.isnan(o[1]) and np.isnan(o[2])


def test_kl_pass_adapted_against_frozen_base_layer():
    """A dense layer's outputs as logits over its N output channels: the
    log-probability difference between the adapted layer (oft_linear_fwd)
    and the reference policy (oft_linear_fwd_base, the frozen base alone)
    against the oracle's, and exactly zero when the adapter is at Q = 0."""
    import torch
    import orthogonal_fine_tuning_amd as oft

    cfg = DenseConfig("kl", M=200, K=512, segs=(256, 256), b=32, x_dtype="bf16", w_fmt="int4", g=64, q_std=0.1)
    inp = make_dense(cfg, seed=8)
    d = oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, oft.OFT_DT_BF16, oft.OFT_W_INT4, cfg.g)
    x, wc, ws = dev(inp["x"]), dev(inp["w_codes"]), dev(inp["w_scales"])
    lab = np.random.default_rng(3).integers(0, cfg.N, cfg.M).astype(np.int32)

    def logits(p):
        Rf = torch.empty((cfg.nblk, cfg.b, cfg.b), dtype=torch.float32, device="cuda")
        Rops = torch.empty((cfg.nblk, 2, cfg.b, cfg.b), dtype=torch.int16, device="cuda")
        oft.cayley_build(dev(p), cfg.nblk, cfg.b, Rf, Rops)
        y = torch.empty((cfg.M, cfg.N), dtype=torch.int16, device="cuda")
        oft.oft_linear_fwd(d, x, wc, ws, Rops, y)
        return y.view(torch.bfloat16).float()  # bf16 logits widened (plumbing)

    yb = torch.empty((cfg.M, cfg.N), dtype=torch.int16, device="cuda")
    oft.oft_linear_fwd_base(d, x, wc, ws, yb)
    ref_logits = yb.view(torch.bfloat16).float()
    out = torch.empty(cfg.M, dtype=torch.float32, device="cuda")
    oft.oft_logprob_diff(logits(inp["p"]), ref_logits, dev(lab), out)
    out0 = torch.empty_like(out)
    oft.oft_logprob_diff(logits(np.zeros_like(inp["p"])), ref_logits, dev(lab), out0)
    torch.cuda.synchronize()
    assert np.all(host(out0) == 0.0)
    W = odense.dequant(inp)
    xo = odense.x_f64(inp)
    want = policy.logprob_diff(odense.forward(xo, W, odense.cayley(inp["p"], cfg.b)), odense.base_forward(xo, W), lab)
    e = err(host(out), want)
    print(f"[kl pass] err={e:.2e} (max |d| {np.abs(want).max():.3f})", flush=True)
    assert e <= 2e-2
