"""MoE layer with OFT on the split gate/up projection, in fp64.

Test infrastructure only (see the package header).

Follows [P1] "Technical details" and [P2] "Dedicated optimisation for
low-precision MoE models": only the experts the router selects are
dequantised, grouped into fixed-size batches ("chunks") of active experts,
and run as a grouped GEMM.  The chunked schedule reaches the plain mixture

    y[t] = sum_{j<k} w[t, j] * W_d,e . SwiGLU(rot_{R_e}(W_gu,e . x[t])),
    e = idx[t, j],

which is what this module evaluates, expert by expert in chunk order.

Readings (the pages print no formula):
  * router: the k largest fp32 logits of a token, in descending order, ties
    to the lower expert index; combine weight w = softmax over all E logits
    evaluated at the selected experts, not renormalised (``renorm=True``
    renormalises over the k selected);
  * grouping: counts per expert, exclusive-scan offsets, a stable
    permutation ordered by (expert, token); perm[pos] = t*k + j and
    inv_perm[t*k + j] = pos; active experts are those with a nonzero count,
    in ascending id; chunk c holds active experts [c*C, (c+1)*C);
  * per expert: gate rows [0, I) and up rows [I, 2I) of W_gu,e; every expert
    has its own adapter, 2I/b blocks, gate blocks first; down has no adapter;
  * SwiGLU(h) = silu(h_gate) * h_up with silu(v) = v / (1 + exp(-v)); no
    clamping;
  * backward returns dX through the experts, dp per expert (zero for
    inactive experts) and dw = dL/dw[t, j] = <dy[t], W_d,e . act>; the
    router logits receive no gradient here.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .codec import bf16_bits_to_f64
from .dense import cayley, cayley_grad, cayley_params, dequant_fmt, rotate, rotate_adjoint, rotation_grad


# ---------------------------------------------------------------- routing
def route(logits: np.ndarray, k: int, renorm: bool = False):
    """Top-k selection and combine weights.

    Selection compares the fp32 logits; k rounds of "largest value, lowest
    index among equals" give the descending order with ties to the lower id.
    """
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    idx = np.empty((T, k), dtype=np.int32)
    work = L.astype(np.float64).copy()
    for j in range(k):
        a = np.argmax(work, axis=1)  # first occurrence = lowest index
        idx[:, j] = a
        work[np.arange(T), a] = -np.inf
    Ld = L.astype(np.float64)
    mx = Ld.max(axis=1, keepdims=True)
    ex = np.exp(Ld - mx)
    w = np.take_along_axis(ex, idx, axis=1) / ex.sum(axis=1, keepdims=True)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w


def router_backward(logits: np.ndarray, idx: np.ndarray, dw: np.ndarray, renorm: bool = False) -> np.ndarray:
    """Gradient of the loss with respect to the router logits, given its
    gradient dw[t, j] with respect to the combine weights w[t, j] of route()
    (the selection idx is held fixed: top-k is piecewise constant).

    Without renormalisation w_j = p[idx_j] with p = softmax over all E, and
    dp_i / dl_e = p_i (delta_ie - p_e), so
        dl_e = p_e (g_e - S),  g_e = dw_j where idx_j = e (else 0),
                               S = sum_j dw_j w_j.
    With renormalisation w is the softmax of the selected logits alone (the
    full denominator cancels), so only selected experts move:
        dl_{idx_m} = w_m (dw_m - S), 0 elsewhere.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    _, w = route(logits, idx.shape[1], renorm=renorm)
    dw = np.asarray(dw, dtype=np.float64)
    S = (dw * w).sum(axis=1, keepdims=True)
    rows = np.arange(T)[:, None]
    out = np.zeros((T, E))
    if renorm:
        out[rows, idx] = w * (dw - S)
    else:
        p = np.exp(L - L.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        g = np.zeros((T, E))
        g[rows, idx] = dw
        out = p * (g - S)
    return out


def group(idx: np.ndarray, E: int, chunk: int) -> dict:
    """Histogram, offsets, stable permutation, active list and chunk table."""
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.empty(T * k, dtype=np.int64)
    for e in range(E):
        # flat pair ids t*k + j selecting e, ascending => ascending token
        sel = np.nonzero(flat == e)[0]
        perm[offsets[e]:offsets[e + 1]] = sel
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(T * k)
    active = np.nonzero(counts)[0]
    chunk_of_expert = np.full(E, -1, dtype=np.int64)
    chunk_of_expert[active] = np.arange(active.size) // chunk
    chunks = [active[i:i + chunk] for i in range(0, active.size, chunk)]
    return dict(counts=counts, offsets=offsets, perm=perm, inv_perm=inv_perm,
                active=active, n_active=int(active.size),
                chunk_of_expert=chunk_of_expert, chunks=chunks)


# ---------------------------------------------------------------- experts
def silu(v):
    return v / (1.0 + np.exp(-v))


def expert_weights(inp: dict, e: int, P=None):
    """Dequantised gate/up [2I, H], down [H, I] and adapter R [2I/b, b, b].

    ``P`` optionally overrides the bf16 adapter parameters with fp64 values
    [E, 2I/b, b(b-1)/2] (used by finite-difference checks).
    """
    cfg = inp["cfg"]
    Wgu = dequant_fmt(cfg.w_fmt, inp["wgu_codes"][e], inp["wgu_scales"][e], cfg.g)
    Wd = dequant_fmt(cfg.w_fmt, inp["wd_codes"][e], inp["wd_scales"][e], cfg.g)
    R = cayley(inp["p"][e], cfg.b) if P is None else cayley_params(P[e], cfg.b)
    return Wgu, Wd, R


def expert_forward(X: np.ndarray, Wgu, Wd, R, I: int):
    """Rows X [n, H] through one expert: (Z, Hh, act, O)."""
    Z = X @ Wgu.T
    Hh = rotate(Z, R)
    act = silu(Hh[:, :I]) * Hh[:, I:]
    return Z, Hh, act, act @ Wd.T


def _pmap(fn, items, threads):
    if threads <= 1:
        return [fn(it) for it in items]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def forward(inp: dict, rt: dict | None = None, experts=None, threads: int = 1,
            X=None, P=None):
    """Chunked evaluation.  Returns (y [T,H], Hsave [P, 2I] permuted, rt).

    ``experts`` restricts the work to a subset (rows of other experts stay
    zero); the full layer uses every active expert.  ``X`` / ``P`` override
    the bf16 activations / adapter parameters with fp64 values.
    """
    cfg = inp["cfg"]
    T, k, H, I = cfg.T, cfg.k, cfg.H, cfg.I
    if rt is None:
        idx, w = route(inp["logits"], k)
        rt = group(idx, cfg.E, cfg.chunk)
        rt.update(idx=idx, w=w)
    if X is None:
        X = bf16_bits_to_f64(inp["x"])
    wflat = rt["w"].reshape(-1)
    order = [int(e) for c in rt["chunks"] for e in c]
    if experts is not None:
        keep = set(int(e) for e in experts)
        order = [e for e in order if e in keep]

    def one(e):
        lo, hi = rt["offsets"][e], rt["offsets"][e + 1]
        pairs = rt["perm"][lo:hi]
        Wgu, Wd, R = expert_weights(inp, e, P)
        _, Hh, _, O = expert_forward(X[pairs // k], Wgu, Wd, R, I)
        return e, Hh, O

    y = np.zeros((T, H))
    Hsave = np.zeros((T * k, 2 * I))
    for e, Hh, O in _pmap(one, order, threads):
        lo, hi = rt["offsets"][e], rt["offsets"][e + 1]
        pairs = rt["perm"][lo:hi]
        Hsave[lo:hi] = Hh
        np.add.at(y, pairs // k, wflat[pairs][:, None] * O)
    return y, Hsave, rt


def expert_backward(inp: dict, e: int, pairs, X, dy, wflat, P=None):
    """Backward of one expert over the given routed pairs (flat ids t*k + j).

    Returns (dw [n], dp [2I/b, b(b-1)/2], dXp [n, H]); dp covers only the
    given pairs (all of the expert's pairs give its full gradient).
    """
    cfg = inp["cfg"]
    k, I, b = cfg.k, cfg.I, cfg.b
    pairs = np.asarray(pairs, dtype=np.int64)
    t = pairs // k
    Wgu, Wd, R = expert_weights(inp, e, P)
    Z, Hh, act, _ = expert_forward(X[t], Wgu, Wd, R, I)
    dA_u = dy[t] @ Wd  # d act before the combine weight
    dw = np.sum(dA_u * act, axis=1)
    dA = wflat[pairs][:, None] * dA_u
    hg, hu = Hh[:, :I], Hh[:, I:]
    sg = 1.0 / (1.0 + np.exp(-hg))
    dH = np.concatenate([dA * hu * sg * (1.0 + hg * (1.0 - sg)), dA * hg * sg], axis=1)
    dp = cayley_grad(R, rotation_grad(dH, Z, b))
    dXp = rotate_adjoint(dH, R) @ Wgu
    return dw, dp, dXp


def backward(inp: dict, rt: dict, experts=None, threads: int = 1, X=None, P=None):
    """Returns (dX [T,H], dp [E, 2I/b, b(b-1)/2], dw [T,k])."""
    cfg = inp["cfg"]
    T, k, H = cfg.T, cfg.k, cfg.H
    if X is None:
        X = bf16_bits_to_f64(inp["x"])
    dy = bf16_bits_to_f64(inp["dy"])
    wflat = rt["w"].reshape(-1)
    order = [int(e) for e in rt["active"]]
    if experts is not None:
        keep = set(int(e) for e in experts)
        order = [e for e in order if e in keep]

    def one(e):
        pairs = rt["perm"][rt["offsets"][e]:rt["offsets"][e + 1]]
        dwe, dpe, dXp = expert_backward(inp, e, pairs, X, dy, wflat, P)
        return e, pairs, dwe, dpe, dXp

    dX = np.zeros((T, H))
    dp_all = np.zeros((cfg.E, cfg.nblk_e, cfg.npair))
    dw = np.zeros(T * k)
    for e, pairs, dwe, dpe, dXp in _pmap(one, order, threads):
        dw[pairs] = dwe
        dp_all[e] = dpe
        np.add.at(dX, pairs // k, dXp)
    return dX, dp_all, dw.reshape(T, k)


def base_forward(inp: dict, rt: dict | None = None):
    """The frozen base alone, the reference policy of [P2] "Five design
    features" (no copy of the actor: the base without the adapter):
    y[t] = sum_j w[t, j] * W_d,e . SwiGLU(W_gu,e . x[t]), e = idx[t, j], the
    gate/up output not rotated.  Returns (y [T, H], Z [P, 2I] in permuted
    order, rt)."""
    cfg = inp["cfg"]
    T, k, H, I = cfg.T, cfg.k, cfg.H, cfg.I
    if rt is None:
        idx, w = route(inp["logits"], k)
        rt = group(idx, cfg.E, cfg.chunk)
        rt.update(idx=idx, w=w)
    X = bf16_bits_to_f64(inp["x"])
    wflat = rt["w"].reshape(-1)
    y = np.zeros((T, H))
    Zs = np.zeros((T * k, 2 * I))
    for e in rt["active"]:
        e = int(e)
        lo, hi = rt["offsets"][e], rt["offsets"][e + 1]
        pairs = rt["perm"][lo:hi]
        Wgu = dequant_fmt(cfg.w_fmt, inp["wgu_codes"][e], inp["wgu_scales"][e], cfg.g)
        Wd = dequant_fmt(cfg.w_fmt, inp["wd_codes"][e], inp["wd_scales"][e], cfg.g)
        Z = X[pairs // k] @ Wgu.T
        act = silu(Z[:, :I]) * Z[:, I:]
        Zs[lo:hi] = Z
        np.add.at(y, pairs // k, wflat[pairs][:, None] * (act @ Wd.T))
    return y, Zs, rt


def bruteforce_forward(inp: dict, idx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Every token through every expert with gate w[t, j] if selected else 0.

    No routing tables, permutation or chunking: the plain mixture.
    """
    cfg = inp["cfg"]
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    X = bf16_bits_to_f64(inp["x"])
    y = np.zeros((T, H))
    for e in range(E):
        Wgu, Wd, R = expert_weights(inp, e)
        gate = np.zeros(T)
        for t in range(T):
            for j in range(cfg.k):
                if idx[t, j] == e:
                    gate[t] = w[t, j]
        _, _, _, O = expert_forward(X, Wgu, Wd, R, I)
        y += gate[:, None] * O
    return y
