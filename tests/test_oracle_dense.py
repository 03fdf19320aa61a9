"""Pins for the dense oracle: closed forms, invariants and finite differences."""
import math

import numpy as np
import pytest

from oft_inputs import CONFIGS, make_dense
from oracle import codec, dense


def _rand_p(rng, nblk, b, std):
    return rng.normal(0.0, std, size=(nblk, b * (b - 1) // 2))


@pytest.mark.parametrize("b", [2, 4, 16, 32])
@pytest.mark.parametrize("std", [0.01, 0.02, 0.5])
def test_cayley_orthogonal_det_one(b, std):
    rng = np.random.default_rng(b * 100 + int(std * 1000))
    R = dense.cayley_params(_rand_p(rng, 24, b, std), b)
    eye = np.eye(b)
    err = np.abs(np.swapaxes(R, 1, 2) @ R - eye).max()
    assert err <= 1e-10
    assert np.allclose(np.linalg.det(R), 1.0, atol=1e-10)


def test_cayley_zero_is_identity_exactly():
    R = dense.cayley_params(np.zeros((5, 16 * 15 // 2)), 16)
    assert np.array_equal(R, np.broadcast_to(np.eye(16), R.shape))


def test_cayley_negated_params_give_transpose():
    rng = np.random.default_rng(3)
    p = _rand_p(rng, 6, 8, 0.3)
    assert np.allclose(dense.cayley_params(-p, 8), np.swapaxes(dense.cayley_params(p, 8), 1, 2),
                       atol=1e-13)


@pytest.mark.parametrize("p", [0.0, 0.01, -0.3, 1.0, 2.5])
def test_cayley_b2_closed_form(p):
    # Q = [[0, p], [-p, 0]]  =>  R = [[cos t, sin t], [-sin t, cos t]], t = 2 atan p
    t = 2.0 * math.atan(p)
    R = dense.cayley_params(np.array([[p]]), 2)[0]
    want = np.array([[math.cos(t), math.sin(t)], [-math.sin(t), math.cos(t)]])
    assert np.allclose(R, want, atol=1e-15)


def test_cayley_single_pair_is_givens():
    b, i, l, p = 8, 2, 5, 0.7
    iu, ju = np.triu_indices(b, 1)
    params = np.zeros((1, iu.size))
    params[0, np.nonzero((iu == i) & (ju == l))[0][0]] = p
    R = dense.cayley_params(params, b)[0]
    t = 2.0 * math.atan(p)
    want = np.eye(b)
    want[i, i] = want[l, l] = math.cos(t)
    want[i, l] = math.sin(t)
    want[l, i] = -math.sin(t)
    assert np.allclose(R, want, atol=1e-15)


def test_rotation_direction_convention():
    # one pair (0, 1) with p > 0 and z = e_1: y_0 = sin(2 atan p) (y = R z)
    p = 0.4
    b = 4
    params = np.zeros((1, 6))
    params[0, 0] = p  # pair (0, 1)
    R = dense.cayley_params(params, b)
    z = np.array([[0.0, 1.0, 0.0, 0.0]])
    y = dense.rotate(z, R)
    t = 2.0 * math.atan(p)
    assert np.allclose(y, [[math.sin(t), math.cos(t), 0.0, 0.0]], atol=1e-15)


def test_packing_order_row_major_upper_triangle():
    b = 4
    params = np.arange(1, 7, dtype=np.float64)[None, :]
    Q = dense.skew(params, b)[0]
    want = np.array([[0, 1, 2, 3], [-1, 0, 4, 5], [-2, -4, 0, 6], [-3, -5, -6, 0]], dtype=float)
    assert np.array_equal(Q, want)


def _tiny_inputs():
    cfg = CONFIGS["tiny_qkv"]
    return cfg, make_dense(cfg, seed=0)


def test_q_zero_reproduces_base_output_exactly():
    cfg, inp = _tiny_inputs()
    W = dense.dequant(inp)
    x = dense.x_f64(inp)
    R = dense.cayley(np.zeros_like(inp["p"]), cfg.b)
    assert np.array_equal(dense.forward(x, W, R), x @ W.T)


def test_fp8_q_zero_reproduces_base_output_exactly():
    cfg = CONFIGS["qkv_4b"].with_(M=32, K=128, segs=(64, 32, 32))
    inp = make_dense(cfg, seed=5)
    W = dense.dequant(inp)
    x = dense.x_f64(inp)
    R = dense.cayley(np.zeros_like(inp["p"]), cfg.b)
    assert np.array_equal(dense.forward(x, W, R), x @ W.T)


def _fp8_golden():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "fp8_channel_scale.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    n = np.array([int(r[0]) for r in rows])
    s = np.array([int(r[1], 16) for r in rows], dtype=np.uint32).view(np.float32)
    c = np.array([int(r[2], 16) for r in rows], dtype=np.uint8)
    v = np.array([float(r[3]) for r in rows])
    return n, s, c, v


def test_fp8_channel_scale_golden():
    """The per-channel scale multiplies the decoded code of its own row (the
    golden table: products of OCP E4M3 values and fp32 scales)."""
    n, s, c, v = _fp8_golden()
    rows = int(n.max()) + 1
    scales = np.zeros(rows, dtype=np.float32)
    scales[n] = s
    # one code per column, on its own row, the other rows' entries zero
    codes = np.zeros((rows, n.size), dtype=np.uint8)
    codes[n, np.arange(n.size)] = c
    W = dense.dequant_fp8(codes, scales)
    got = W[n, np.arange(n.size)]
    assert np.array_equal(got, v) and np.array_equal(np.signbit(got), np.signbit(v))


def _fp8_source_weights(cfg, seed):
    """The generator's fp32 weights before quantisation (same seeded stream:
    x is drawn first, then w ~ N(0, 1))."""
    rng = np.random.default_rng(seed)
    rng.standard_normal((cfg.M, cfg.K), dtype=np.float32)
    return rng.standard_normal((cfg.N, cfg.K), dtype=np.float32).astype(np.float64)


def _fp8_reconstructs(W, w, s):
    # e4m3fn keeps 3 fraction bits: a normal value is within 2^-4 relative
    # of what was encoded; below 2^-6 the spacing is 2^-9, so the absolute
    # error is at most 2^-10 (times the row scale)
    tol = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s[:, None])
    return bool(np.all(np.abs(W - w) <= tol * (1 + 1e-12)))


def test_fp8_dequant_reconstructs_generator_weights():
    """code * s[n] gives back the generator's w to e4m3 rounding (w / s was
    encoded, s[n] = max_k |w[n, k]| / 448); dividing by the scale, or taking
    it along the wrong axis, does not (planted mistakes)."""
    cfg = CONFIGS["qkv_4b"].with_(M=8, K=192, segs=(96, 64, 32))
    inp = make_dense(cfg, seed=3)
    w = _fp8_source_weights(cfg, 3)
    s = np.asarray(inp["w_scales"], dtype=np.float64)
    assert _fp8_reconstructs(dense.dequant(inp), w, s)
    e = dense.dequant_fp8_codes(inp["w_codes"])
    wrong = {"divided by the scale": e / s[:, None],
             "scale of another row": e * np.roll(s, 1)[:, None],
             "scale along the in-features": e * np.resize(s, cfg.K)[None, :]}
    for name, Wb in wrong.items():
        assert not _fp8_reconstructs(Wb, w, s), name


def test_base_forward_is_the_q_zero_layer():
    """The reference-policy layer (frozen base alone) is the adapted layer at
    Q = 0 exactly, and differs from it once the adapter has moved."""
    for cfg, inp in (_tiny_inputs(),
                     (lambda c: (c, make_dense(c, seed=5)))(CONFIGS["qkv_4b"].with_(M=32, K=128, segs=(64, 32, 32)))):
        W = dense.dequant(inp)
        x = dense.x_f64(inp)
        yb = dense.base_forward(x, W)
        assert np.array_equal(yb, dense.forward(x, W, dense.cayley(np.zeros_like(inp["p"]), cfg.b)))
        y = dense.forward(x, W, dense.cayley(inp["p"], cfg.b))
        assert np.abs(y - yb).max() > 1e-3 * np.abs(yb).max()


def test_forward_preserves_block_norms_and_is_linear():
    cfg, inp = _tiny_inputs()
    W = dense.dequant(inp)
    x = dense.x_f64(inp)
    R = dense.cayley(inp["p"], cfg.b)
    Z = x @ W.T
    Y = dense.forward(x, W, R)
    nz = np.linalg.norm(Z.reshape(cfg.M, -1, cfg.b), axis=2)
    ny = np.linalg.norm(Y.reshape(cfg.M, -1, cfg.b), axis=2)
    assert np.allclose(nz, ny, rtol=1e-12)
    rng = np.random.default_rng(7)
    x2 = rng.standard_normal(x.shape)
    assert np.allclose(dense.forward(2.0 * x - 3.0 * x2, W, R), 2.0 * Y - 3.0 * dense.forward(x2, W, R),
                       atol=1e-11)


def test_rotation_acts_per_block_only():
    # changing the parameters of block j changes only the columns of block j
    cfg, inp = _tiny_inputs()
    W = dense.dequant(inp)
    x = dense.x_f64(inp)
    p = codec.bf16_bits_to_f64(inp["p"])
    p2 = p.copy()
    p2[5] += 0.1
    Y1 = dense.forward(x, W, dense.cayley_params(p, cfg.b))
    Y2 = dense.forward(x, W, dense.cayley_params(p2, cfg.b))
    diff = np.abs(Y1 - Y2).max(axis=0)
    blk = np.arange(cfg.N) // cfg.b
    assert np.all(diff[blk != 5] == 0.0)
    assert np.all(diff[blk == 5] > 0.0)


def test_adjoint_identity():
    cfg, inp = _tiny_inputs()
    W = dense.dequant(inp)
    x = dense.x_f64(inp)
    R = dense.cayley(inp["p"], cfg.b)
    dY = codec.bf16_bits_to_f64(inp["dy"])
    y = dense.forward(x, W, R)
    dX, _ = dense.backward(x, W, R, dY)
    lhs, rhs = np.sum(dY * y), np.sum(dX * x)
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0) * 10


def _small_problem(seed=11):
    rng = np.random.default_rng(seed)
    M, K, b = 5, 6, 8
    N = 16  # two segments of one block each
    x = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K))
    p = _rand_p(rng, N // b, b, 0.3)
    dY = rng.standard_normal((M, N))
    return x, W, p, dY, b


def test_dx_central_difference():
    x, W, p, dY, b = _small_problem()
    R = dense.cayley_params(p, b)
    dX, _ = dense.backward(x, W, R, dY)
    h = 1e-6
    num = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        num[idx] = (np.sum(dY * dense.forward(xp, W, R)) - np.sum(dY * dense.forward(xm, W, R))) / (2 * h)
    assert np.abs(num - dX).max() <= 1e-7 * np.abs(dX).max()


def test_dp_central_difference():
    x, W, p, dY, b = _small_problem(12)
    R = dense.cayley_params(p, b)
    _, dp = dense.backward(x, W, R, dY)
    h = 1e-6
    num = np.zeros_like(p)
    for idx in np.ndindex(*p.shape):
        pp, pm = p.copy(), p.copy()
        pp[idx] += h
        pm[idx] -= h
        lp = np.sum(dY * dense.forward(x, W, dense.cayley_params(pp, b)))
        lm = np.sum(dY * dense.forward(x, W, dense.cayley_params(pm, b)))
        num[idx] = (lp - lm) / (2 * h)
    assert np.abs(num - dp).max() <= 1e-7 * np.abs(dp).max()


def test_dp_at_q_zero_closed_form():
    # R = I  =>  dL/dQ = 2 G, dp_il = 2 (G_il - G_li) with G = dY_blk^T Z_blk
    x, W, p, dY, b = _small_problem(13)
    R = dense.cayley_params(np.zeros_like(p), b)
    _, dp = dense.backward(x, W, R, dY)
    Z = x @ W.T
    iu, ju = np.triu_indices(b, 1)
    for j in range(p.shape[0]):
        G = dY[:, j * b:(j + 1) * b].T @ Z[:, j * b:(j + 1) * b]
        assert np.allclose(dp[j], 2.0 * (G[iu, ju] - G[ju, iu]), atol=1e-13)


def test_run_tiny_config_shapes():
    cfg, inp = _tiny_inputs()
    out = dense.run(inp)
    assert out["y"].shape == (cfg.M, cfg.N)
    assert out["dx"].shape == (cfg.M, cfg.K)
    assert out["dp"].shape == (cfg.nblk, cfg.npair)
    assert np.all(np.isfinite(out["y"]))


# ---- the pins catch plausible mistakes (mistakes planted in the oracle, CPU only)
def test_planted_mistakes_fail_the_pins(monkeypatch):
    x, W, p, dY, b = _small_problem(14)
    h = 1e-6

    def fd_dp(R_of_p):
        num = np.zeros_like(p)
        for idx in np.ndindex(*p.shape):
            pp, pm = p.copy(), p.copy()
            pp[idx] += h
            pm[idx] -= h
            num[idx] = (np.sum(dY * dense.forward(x, W, R_of_p(pp)))
                        - np.sum(dY * dense.forward(x, W, R_of_p(pm)))) / (2 * h)
        return num

    num = fd_dp(lambda q: dense.cayley_params(q, b))
    R = dense.cayley_params(p, b)
    G = dense.rotation_grad(dY, x @ W.T, b)
    eye = np.eye(b)
    Rt = np.swapaxes(R, 1, 2) + eye
    wrong = {
        "no half": dense.pack_skew_grad(Rt @ G @ Rt),
        "R instead of R^T": dense.pack_skew_grad(0.5 * ((R + eye) @ G @ (R + eye))),
        "G transposed": dense.pack_skew_grad(0.5 * (Rt @ np.swapaxes(G, 1, 2) @ Rt)),
        "sign of skew pack": -dense.cayley_grad(R, G),
    }
    for name, dp in wrong.items():
        assert np.abs(num - dp).max() > 1e-3 * np.abs(num).max(), name
    # a transposed rotation in the forward breaks the direction pin
    params = np.zeros((1, 6))
    params[0, 0] = 0.4
    Rr = dense.cayley_params(params, 4)
    y_wrong = np.array([[0.0, 1.0, 0.0, 0.0]]) @ Rr[0]
    assert not np.allclose(y_wrong, [[math.sin(2 * math.atan(0.4)), math.cos(2 * math.atan(0.4)), 0, 0]])
