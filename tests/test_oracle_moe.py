"""Pins for the MoE oracle: library sorting, invariants, brute force, FD."""
import numpy as np
import pytest

from oft_inputs import CONFIGS, MoEConfig, make_moe
from oracle import codec, moe

TINY = MoEConfig("tiny_moe", T=32, E=8, k=2, H=64, I=32, g=32, chunk=3, b=8, q_std=0.2)


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((500, 40)).astype(np.float32)
    # plant ties: duplicate some logits inside rows
    L[::7, 5] = L[::7, 9]
    L[::11, 3] = L[::11, 1]
    L[0, :] = 1.0  # all equal: must select 0..k-1
    idx, _ = moe.route(L, 6)
    ref = np.argsort(-L, axis=1, kind="stable")[:, :6]
    assert np.array_equal(idx, ref)
    assert idx[0].tolist() == [0, 1, 2, 3, 4, 5]


def test_softmax_weights():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((64, 16)).astype(np.float32)
    idx, w = moe.route(L, 4)
    full = np.exp(L.astype(np.float64))
    full /= full.sum(axis=1, keepdims=True)
    assert np.allclose(w, np.take_along_axis(full, idx, axis=1), rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all(w.sum(axis=1) < 1.0)
    _, wn = moe.route(L, 4, renorm=True)
    assert np.allclose(wn.sum(axis=1), 1.0)


def test_grouping_invariants():
    rng = np.random.default_rng(6)
    T, E, k, C = 300, 24, 4, 5
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:, 3] -= 100.0  # expert 3 never selected -> inactive
    idx, _ = moe.route(L, k)
    rt = moe.group(idx, E, C)
    assert rt["counts"].sum() == T * k
    assert np.array_equal(rt["offsets"][1:], np.cumsum(rt["counts"]))
    assert np.array_equal(np.sort(rt["perm"]), np.arange(T * k))
    assert np.array_equal(rt["perm"][rt["inv_perm"]], np.arange(T * k))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = rt["perm"][rt["offsets"][e]:rt["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)  # stable: ascending token
    assert 3 not in rt["active"]
    assert rt["n_active"] == E - 1
    assert np.all(np.diff(rt["active"]) > 0)
    assert rt["chunk_of_expert"][3] == -1
    assert [len(c) for c in rt["chunks"]] == [5, 5, 5, 5, 3]


def test_bruteforce_matches_chunked_forward():
    inp = make_moe(TINY, seed=0)
    y, _, rt = moe.forward(inp)
    yb = moe.bruteforce_forward(inp, rt["idx"], rt["w"])
    assert np.abs(y - yb).max() <= 1e-12 * np.abs(yb).max()


def test_chunk_size_invariance():
    inp = make_moe(TINY, seed=1)
    ys = []
    for C in (1, 3, TINY.E):
        y, _, _ = moe.forward({**inp, "cfg": TINY.with_(chunk=C)})
        ys.append(y)
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_per_token_loop_matches_grouped():
    inp = make_moe(TINY, seed=2)
    y, _, rt = moe.forward(inp)
    X = codec.bf16_bits_to_f64(inp["x"])
    for t in (0, 7, 31):
        acc = np.zeros(TINY.H)
        for j in range(TINY.k):
            Wgu, Wd, R = moe.expert_weights(inp, int(rt["idx"][t, j]))
            _, _, _, O = moe.expert_forward(X[t:t + 1], Wgu, Wd, R, TINY.I)
            acc += rt["w"][t, j] * O[0]
        assert np.allclose(acc, y[t], atol=1e-12)


def _loss(inp, rt, X=None, P=None, w=None):
    rt2 = dict(rt)
    if w is not None:
        rt2["w"] = w
    y, _, _ = moe.forward(inp, rt2, X=X, P=P)
    return np.sum(codec.bf16_bits_to_f64(inp["dy"]) * y)


def test_moe_gradients_central_difference():
    cfg = TINY.with_(T=6, E=4, H=64, I=32, chunk=2)
    inp = make_moe(cfg, seed=3)
    _, _, rt = moe.forward(inp)
    X = codec.bf16_bits_to_f64(inp["x"])
    P = codec.bf16_bits_to_f64(inp["p"])
    dX, dP, dw = moe.backward(inp, rt)
    h = 1e-6
    rng = np.random.default_rng(0)
    # dX on a sample of entries
    for _ in range(12):
        t, c = rng.integers(cfg.T), rng.integers(cfg.H)
        Xp, Xm = X.copy(), X.copy()
        Xp[t, c] += h
        Xm[t, c] -= h
        num = (_loss(inp, rt, X=Xp) - _loss(inp, rt, X=Xm)) / (2 * h)
        assert abs(num - dX[t, c]) <= 1e-6 * max(1.0, np.abs(dX).max())
    # dp on a sample of entries of active experts
    for _ in range(12):
        e = int(rng.choice(rt["active"]))
        j, q = rng.integers(cfg.nblk_e), rng.integers(cfg.npair)
        Pp, Pm = P.copy(), P.copy()
        Pp[e, j, q] += h
        Pm[e, j, q] -= h
        num = (_loss(inp, rt, P=Pp) - _loss(inp, rt, P=Pm)) / (2 * h)
        assert abs(num - dP[e, j, q]) <= 1e-6 * max(1.0, np.abs(dP).max())
    # dw: the loss is linear in w
    for t in range(cfg.T):
        for j in range(cfg.k):
            wp = rt["w"].copy()
            wp[t, j] += 1.0
            num = _loss(inp, rt, w=wp) - _loss(inp, rt)
            assert abs(num - dw[t, j]) <= 1e-9 * max(1.0, np.abs(dw).max())
    # inactive experts get exactly zero
    inactive = [e for e in range(cfg.E) if e not in set(rt["active"].tolist())]
    for e in inactive:
        assert np.all(dP[e] == 0.0)


@pytest.mark.parametrize("name", ["moe_30b_a3b", "moe_1t_train"])
def test_routing_on_config_logits(name):
    """Routing of the real config logits (no weights needed)."""
    cfg = CONFIGS[name]
    rng = np.random.default_rng(0)
    # regenerate only the logits with the generator's draw order
    rng.standard_normal((cfg.T, cfg.H), dtype=np.float32)
    L = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.bias_std > 0:
        L = (L + rng.normal(0.0, cfg.bias_std, size=cfg.E).astype(np.float32)[None, :]).astype(np.float32)
    idx, w = moe.route(L, cfg.k)
    assert np.array_equal(idx, np.argsort(-L, axis=1, kind="stable")[:, :cfg.k])
    rt = moe.group(idx, cfg.E, cfg.chunk)
    assert rt["counts"].sum() == cfg.P


def _router_case(seed, T=24, E=12, k=3):
    """Distinct logits on a 1/64 grid, so that a step of 2^-10 is exact in
    fp32 and never changes the top-k selection."""
    rng = np.random.default_rng(seed)
    L = np.stack([rng.permutation(np.arange(-E, E)[:E]) for _ in range(T)]).astype(np.float64) * (5.0 / 64)
    L = L.astype(np.float32)
    dw = rng.standard_normal((T, k))
    return L, dw


@pytest.mark.parametrize("renorm", [False, True])
def test_router_backward_central_difference(renorm):
    L, dw = _router_case(11)
    T, E = L.shape
    k = dw.shape[1]
    idx, _ = moe.route(L, k, renorm=renorm)
    g = moe.router_backward(L, idx, dw, renorm=renorm)
    h = 2.0 ** -10
    fd = np.zeros_like(g)
    for e in range(E):
        Lp, Lm = L.copy(), L.copy()
        Lp[:, e] += np.float32(h)
        Lm[:, e] -= np.float32(h)
        ip, wp = moe.route(Lp, k, renorm=renorm)
        im, wm = moe.route(Lm, k, renorm=renorm)
        assert np.array_equal(ip, idx) and np.array_equal(im, idx)
        fd[:, e] = ((dw * wp).sum(axis=1) - (dw * wm).sum(axis=1)) / (2 * h)
    assert np.abs(g - fd).max() <= 1e-5 * np.abs(g).max()


@pytest.mark.parametrize("renorm", [False, True])
def test_router_backward_rows_sum_to_zero(renorm):
    # adding a constant to every logit of a token changes no weight
    L, dw = _router_case(12, T=40, E=16, k=4)
    idx, _ = moe.route(L, 4, renorm=renorm)
    g = moe.router_backward(L, idx, dw, renorm=renorm)
    assert np.abs(g.sum(axis=1)).max() <= 1e-12 * np.abs(g).max()
    if renorm:  # only the selected logits enter the renormalised weights
        mask = np.ones_like(g, dtype=bool)
        mask[np.arange(g.shape[0])[:, None], idx] = False
        assert np.all(g[mask] == 0.0)


def test_base_forward_is_the_q_zero_layer_and_differs_otherwise():
    """The reference-policy layer (frozen base, no rotation) equals the
    adapted layer at Q = 0 (R = I exactly) and differs once Q moves; its
    saved gate/up output is the un-rotated Z."""
    cfg = MoEConfig("base", T=48, E=6, k=2, H=64, I=32, g=32, chunk=2, b=8, q_std=0.2)
    inp = make_moe(cfg, seed=4)
    yb, Zb, rt = moe.base_forward(inp)
    inp0 = dict(inp)
    inp0["p"] = np.zeros_like(inp["p"])
    y0, H0, _ = moe.forward(inp0)
    assert np.array_equal(yb, y0)
    assert np.array_equal(Zb, H0)
    y1, H1, _ = moe.forward(inp)
    assert np.abs(y1 - yb).max() > 1e-3 * np.abs(yb).max()
    # brute force over every expert, gate weights w or 0 (R = I: no rotation)
    ybf = moe.bruteforce_forward(inp0, rt["idx"], rt["w"])
    assert np.abs(yb - ybf).max() <= 1e-12 * np.abs(yb).max()
