#!/usr/bin/env python3
"""Benchmark of the OFT dequant-GEMM hot path on one MI355X.

A step is one pass of the whole path over one batch of a workload: the
Cayley build of the adapter rotations, the forward and the backward (dense:
dX and dQ; MoE: routing, grouped gate/up with the per-expert rotation,
SwiGLU, down, combine, and dX, dQ and the combine-weight gradient dw).
Inputs are seeded synthetic data (``oft_inputs``), resident in HBM before
timing starts.

By default every workload runs: the seven shapes of the OFT layer (fused
Q/K/V of a 4B model, gate/up of a 4B model at a training token count and a
decode batch, the tiny parity shape, a 30B-A3B MoE layer and one GPU's share
of a ~1T MoE layer at a training token count and a decode batch).  The
printed line is the largest single-GPU workload, the ~1T-shaped MoE layer at
4096 tokens (``--config`` picks another, or ``all``); every workload's
figures are under ``workloads``.

Per workload:
  * ``value``: algorithmic TFLOP/s of the whole step (dense fwd 2MNK + 2MNb,
    bwd 2MNK + 4MNb; MoE fwd 2P.H.2I + 2P.I.H + 2P.2I.b, bwd the same GEMMs
    + 4P.2I.b; the Cayley build is timed inside the step but its flops are
    not counted), over the wall time of K steps bracketed by syncs;
  * ``step_roofline``: that step against the bound of its arithmetic
    intensity (algorithmic flop per algorithmic HBM byte): the bf16 matrix
    peak above the ridge point (312.5 flop/B), HBM below it;
  * ``kernels``: the library's per-step kernel times, from HIP events the
    library records on the launch stream around each step of its work
    (``oft_prof_*``), averaged over profiled steps run right after the timed
    ones;
  * ``roofline``: the dominant kernel step (the largest time per step): its
    algorithmic flops or bytes per launch over its average duration, against
    the matrix peak or HBM by its own intensity; ``traffic`` is the HBM
    bytes per launch from committed rocprofv3 counter runs
    (``profiles/traffic.json``), null when the kernel sources changed since;
  * ``cpu_baseline``: the fp64 CPU oracle timed on a bounded sample of the
    workload (token rows for dense layers, a few experts for MoE layers);
  * MoE: ``transient_bytes`` (device memory allocated during the timed calls
    beyond what existed before: the library allocates nothing) and
    ``dense_bf16_reference`` (the same calls on every expert's weights
    dequantised to bf16 beforehand; the ratio of the 4-bit path's time to
    it); dense: ``reference_policy_fwd`` (the frozen base alone) and
    ``slots_fwd`` (the forward on the active slot of a double-buffered
    adapter), timed as bursts of back-to-back launches; ``phases_cold_us``:
    fwd and bwd again, each right after evicting the last-level cache.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "OFT dequant-GEMM fwd+bwd TFLOP/s and HBM GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte where the two meet (312.5)
HEADLINE = "moe_1t_train"
ORDER = ["moe_1t_train", "qkv_4b", "gateup_4b_train", "gateup_4b_decode", "tiny_qkv", "moe_30b_a3b",
         "moe_1t_decode"]
SOURCES = "orthogonal_fine_tuning_amd/csrc"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all", help="a workload name, or 'all' (the default)")
    ap.add_argument("--w-fmt", choices=("int4", "fp4"), default=None,
                    help="run the 4-bit workloads with this base format (FP4: OCP MX E2M1 codes, E8M0 group "
                         "exponents in the same layout and bytes as INT4)")
    ap.add_argument("--storage", choices=("auto", "row-major"), default="auto",
                    help="MoE INT4 weights: 'auto' packs them once, untimed, into the tiled storage "
                         "(OFT_W_INT4_TILED) where H and I are multiples of 256; 'row-major' keeps them as given")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-ref", action="store_true",
                    help="MoE: skip the dense-bf16-weight reference run of the same grouped kernels")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip phases_cold_us (keeps a profiler's kernel averages to the timed steps)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the reference-policy, slot and router-backward bursts")
    ap.add_argument("--prof-steps", type=int, default=5, help="steps timed kernel by kernel after the timed ones")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="about this much oracle work per non-headline workload (3x for the headline)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (a reference "
                         "for HBM byte counters)")
    ap.add_argument("--pmc-summary", metavar="DIR", default=None,
                    help="no GPU work: summarise the rocprofv3 runs under DIR/<workload>/<pass> (see "
                         "pmc_summary) into profiles/")
    return ap.parse_args()


# ------------------------------------------------------------------ rooflines
def roofline(flops, nbytes, seconds, kernel=None, traffic=None):
    """Above the ridge point: algorithmic TFLOP/s against the bf16 matrix
    peak; below it: algorithmic GB/s against HBM."""
    mfma = nbytes == 0 or flops / nbytes > RIDGE
    if mfma:
        achieved, peak, unit = flops / seconds / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / seconds / 1e9, PEAK_HBM_GBS, "GB/s"
    out = {"bound": "mfma" if mfma else "hbm", "achieved": round(achieved, 2), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4)}
    if kernel is not None:
        out["traffic"] = traffic
        out["kernel"] = kernel
    out.update({"us": round(seconds * 1e6, 2), "algorithmic_flops": int(flops), "algorithmic_bytes": int(nbytes)})
    return out


def source_sha():
    h = hashlib.sha256()
    d = os.path.join(ROOT, SOURCES)
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(key, sha):
    """HBM bytes per launch of a kernel step from the committed counter runs,
    or None when the sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get("entries", {}).get(key)
    if not ent or data.get("source_sha") != sha:
        return None
    return ent.get("bytes_per_launch")


def burst_seconds(stream, launch, n=10):
    """Mean duration of one of n back-to-back launches: HIP events on the
    launch stream around the burst, queued behind a short GPU spin so that
    the host's cost per call adds no idle time between the kernels."""
    import torch

    eb = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(2_000_000)  # a bounded spin of one thread: about a millisecond
    eb[0].record(stream)
    for _ in range(n):
        launch()
    eb[1].record(stream)
    torch.cuda.synchronize()
    return eb[0].elapsed_time(eb[1]) * 1e-3 / n


def profile_steps(step, nsteps):
    """Per-step kernel times from the library's own HIP events (averaged over
    nsteps steps): {name: (milliseconds per step, launches per step)}."""
    import torch

    import orthogonal_fine_tuning_amd as oft

    torch.cuda.synchronize()
    oft.prof_enable(True)
    try:
        for _ in range(nsteps):
            step()
        torch.cuda.synchronize()
        recs = oft.prof_records()
    finally:
        oft.prof_enable(False)
    agg = {}
    for name, ms in recs:
        t, c = agg.get(name, (0.0, 0))
        agg[name] = (t + ms, c + 1)
    return {k: (t / nsteps, c / nsteps) for k, (t, c) in agg.items()}


def cold_phases(fwd, bwd, reps=5):
    """fwd and bwd timed separately (HIP events on the current stream), each
    right after writing 512 MiB of device memory, twice the 256 MB
    last-level cache (MALL), so that the weights come from HBM.  Medians in
    seconds."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    tf, tb = [], []
    for i in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        flush.fill_(i & 255)
        ev[0].record(stream)
        fwd()
        ev[1].record(stream)
        flush.fill_((i + 1) & 255)
        ev[2].record(stream)
        bwd()
        ev[3].record(stream)
        torch.cuda.synchronize()
        tf.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        tb.append(ev[2].elapsed_time(ev[3]) * 1e-3)
    del flush
    torch.cuda.empty_cache()
    return float(np.median(tf)), float(np.median(tb))


def blas_threads():
    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        return max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - informational only
        return os.cpu_count() or 1


def time_steps(step, steps, warmup, nev=4):
    """Warm-up, then `steps` steps bracketed by syncs (wall clock, nothing
    else on the stream), then the same number of steps again with HIP events
    between their phases for the phase split (an event record between two
    kernels adds a few microseconds of its own, so it stays out of the timed
    steps)."""
    import numpy as np
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    phases = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e-3 for i in range(nev - 1)]
    return wall / steps, phases


# ------------------------------------------------------------------ dense
def dense_flops(cfg):
    M, N, K, b = cfg.M, cfg.N, cfg.K, cfg.b
    return 2 * M * N * K + 2 * M * N * b, 2 * M * N * K + 4 * M * N * b


def dense_bytes(cfg):
    """Algorithmic HBM bytes: what the method must read and write once."""
    M, N, K, b = cfg.M, cfg.N, cfg.K, cfg.b
    xb = 4 if cfg.x_dtype == "f32" else 2
    wbytes = N * K // 2 + N * (K // cfg.g) * 2 if cfg.w_fmt in ("int4", "fp4") else N * K + N * 4
    nblk = N // b
    rops = nblk * 2 * b * b * 2
    rf = nblk * b * b * 4
    dq = nblk * (b * (b - 1) // 2) * 4
    fwd = wbytes + M * K * xb + M * N * xb + rops
    bwd = wbytes + M * N * 2 + M * N * xb + M * K * xb + rops + rf + dq
    return fwd, bwd, wbytes


def dense_kernel_work(cfg):
    """Algorithmic (flops, bytes) per launch of each kernel step."""
    M, N, K, b = cfg.M, cfg.N, cfg.K, cfg.b
    xb = 4 if cfg.x_dtype == "f32" else 2
    f_fwd, _ = dense_flops(cfg)
    b_fwd, _, wbytes = dense_bytes(cfg)
    nblk = N // b
    return {
        "dense.fwd": (f_fwd, b_fwd),
        "dense.fwd_base": (2 * M * N * K, b_fwd - nblk * 2 * b * b * 2),
        # dX = rot^T(dY) W: the contraction, reading the weight and dZ' once
        "dense.dx": (2 * M * N * K, wbytes + M * N * 2 + M * K * xb),
        # dQ pass: S = dY^T Y per block and the rotated dY (2MNb each),
        # reading dY and Y, writing dZ'
        "dense.dq": (4 * M * N * b, M * N * 2 + M * N * xb + M * N * 2 + nblk * 2 * b * b * 2),
        "dense.dq_final": (4 * nblk * b ** 3, nblk * b * b * 4 * 2 + nblk * (b * (b - 1) // 2) * 4),
        "dense.transpose": (0, wbytes + K * N * (1 if cfg.w_fmt == "fp8" else 2)),
        "dense.dx_reduce": (0, M * K * (4 + xb)),
        "cayley": (2 * nblk * b ** 3, nblk * (b * (b - 1) // 2) * 2 + nblk * b * b * 4 + nblk * 2 * b * b * 2),
    }


def dense_cpu_baseline(cfg, inp, seconds):
    """The oracle on a row sample of about `seconds` of work (one timed pass,
    scaled from a small probe)."""
    from oracle import dense as odense

    def run_rows(m):
        sub = dict(inp)
        sub["cfg"] = cfg.with_(M=m)
        sub["x"] = inp["x"][:m]
        sub["dy"] = inp["dy"][:m]
        t0 = time.perf_counter()
        odense.run(sub)
        return time.perf_counter() - t0, sub["cfg"]

    m = min(cfg.M, 64)
    dt, sc = run_rows(m)
    if m < cfg.M and dt < seconds / 2:
        m = int(min(cfg.M, max(m, m * seconds / max(dt, 1e-3))))
        dt, sc = run_rows(m)
    f, b = dense_flops(sc)
    return {"value": (f + b) / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{cfg.name}: {m} of {cfg.M} token rows, dequant + Cayley + fwd + bwd (dX, dQ) "
                      f"in fp64 numpy, {dt:.2f} s"}


def run_dense(cfg, args, sha, headline):
    import numpy as np
    import torch

    import orthogonal_fine_tuning_amd as oft
    from oft_inputs import make_dense

    inp = make_dense(cfg, seed=0)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    xdt = oft.OFT_DT_F32 if cfg.x_dtype == "f32" else oft.OFT_DT_BF16
    wf = {"int4": oft.OFT_W_INT4, "fp8": oft.OFT_W_FP8_E4M3, "fp4": oft.OFT_W_FP4_E2M1}[cfg.w_fmt]
    d = oft.linear_desc(cfg.M, cfg.K, cfg.segs, cfg.b, xdt, wf, cfg.g)
    tdt = torch.float32 if cfg.x_dtype == "f32" else torch.int16
    q, x = dev(inp["p"]), dev(inp["x"])
    wc, ws = dev(inp["w_codes"]), dev(inp["w_scales"])
    dy = dev(inp["dy"])
    Rf = torch.empty((cfg.nblk, cfg.b, cfg.b), dtype=torch.float32, device="cuda")
    Rops = torch.empty((cfg.nblk, 2, cfg.b, cfg.b), dtype=torch.int16, device="cuda")
    y = torch.empty((cfg.M, cfg.N), dtype=tdt, device="cuda")
    dx = torch.empty((cfg.M, cfg.K), dtype=tdt, device="cuda")
    dq = torch.empty((cfg.nblk, cfg.npair), dtype=torch.float32, device="cuda")
    nb = oft.oft_linear_workspace_bytes(d, oft.OFT_PASS_BWD)
    work = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def fwd():
        oft.oft_linear_fwd(d, x, wc, ws, Rops, y, stream=sp)

    def bwd():
        oft.oft_linear_bwd(d, dy, y, wc, ws, Rf, Rops, dx, dq, work, nb, stream=sp)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        oft.cayley_build(q, cfg.nblk, cfg.b, Rf, Rops, stream=sp)
        if ev is not None:
            ev[1].record(stream)
        fwd()
        if ev is not None:
            ev[2].record(stream)
        bwd()
        if ev is not None:
            ev[3].record(stream)

    t_step, (t_cay, t_fwd, t_bwd) = time_steps(step, args.steps, args.warmup)
    kern = profile_steps(step, args.prof_steps)
    f_fwd, f_bwd = dense_flops(cfg)
    by_fwd, by_bwd, _ = dense_bytes(cfg)
    out = summary(cfg.name, t_step, f_fwd + f_bwd, by_fwd + by_bwd, kern, dense_kernel_work(cfg), sha,
                  {"cayley_build": t_cay, "fwd": t_fwd, "bwd": t_bwd})
    out["config"] = {"workload": cfg.name, "tokens": cfg.M, "in_features": cfg.K, "out_features": cfg.N,
                     "segments": list(cfg.segs), "oft_block": cfg.b,
                     "weights": cfg.w_fmt + (f"_g{cfg.g}" if cfg.w_fmt != "fp8" else "_e4m3"),
                     "x_dtype": cfg.x_dtype, "parallelism": "single_gpu"}
    out["phase_rates"] = {"fwd_tflops": round(f_fwd / t_fwd / 1e12, 2), "bwd_tflops": round(f_bwd / t_bwd / 1e12, 2),
                          "fwd_alg_gbs": round(by_fwd / t_fwd / 1e9, 1), "bwd_alg_gbs": round(by_bwd / t_bwd / 1e9, 1)}
    if not args.no_extras:
        burst = 10
        t_base = burst_seconds(stream, lambda: oft.oft_linear_fwd_base(d, x, wc, ws, y, stream=sp), burst)
        fb, bb = dense_kernel_work(cfg)["dense.fwd_base"]
        out["reference_policy_fwd"] = roofline(fb, bb, t_base)
        state = torch.zeros(4, dtype=torch.int32, device="cuda")
        latch = torch.zeros(4, dtype=torch.int32, device="cuda")
        oft.oft_slots_switch(state, 1, 1, stream=sp)
        ts, tp = [], []
        for _ in range(3):  # alternating bursts, medians (the clock settles under sustained load)
            ts.append(burst_seconds(stream, lambda: oft.oft_linear_fwd_slots(d, x, wc, ws, Rops, Rops, state, latch,
                                                                             y, stream=sp), burst))
            tp.append(burst_seconds(stream, fwd, burst))
        t_s, t_p = float(np.median(ts)), float(np.median(tp))
        out["slots_fwd"] = {"us": round(t_s * 1e6, 2), "plain_fwd_us": round(t_p * 1e6, 2),
                            "overhead_us": round((t_s - t_p) * 1e6, 2)}
    if not args.no_cold:
        cf, cb = cold_phases(fwd, bwd)
        out["phases_cold_us"] = {"fwd": round(cf * 1e6, 2), "bwd": round(cb * 1e6, 2),
                                 "fwd_alg_gbs": round(by_fwd / cf / 1e9, 1), "bwd_alg_gbs": round(by_bwd / cb / 1e9, 1)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = dense_cpu_baseline(cfg, inp, args.cpu_seconds * (3 if headline else 1))
    del x, wc, ws, dy, Rf, Rops, y, dx, dq, work
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ MoE
def moe_flops(cfg):
    P, H, I, b = cfg.T * cfg.k, cfg.H, cfg.I, cfg.b
    gemm = 2 * P * H * 2 * I + 2 * P * I * H
    return gemm + 2 * P * 2 * I * b, gemm + 4 * P * 2 * I * b


def moe_weight_bytes(cfg):
    """Packed bytes of one expert's gate/up and down weights (codes + scales)."""
    H, I, g = cfg.H, cfg.I, cfg.g
    return 2 * I * H // 2 + 2 * I * (H // g) * 2, H * I // 2 + H * (I // g) * 2


def moe_bytes(cfg, n_active):
    P, T, E, H, I, b = cfg.T * cfg.k, cfg.T, cfg.E, cfg.H, cfg.I, cfg.b
    wgu, wd = moe_weight_bytes(cfg)
    nblk = 2 * I // b
    rops = nblk * 2 * b * b * 2
    fwd = n_active * (wgu + wd + rops) + T * H * 2 + T * E * 4 + P * 2 * I * 2 + T * H * 2 + P * 16
    bwd = (n_active * (wgu + wd + rops + nblk * b * b * 4) + T * H * 2 + P * 2 * I * 2 + T * H * 2
           + E * nblk * (b * (b - 1) // 2) * 4 + P * 4 + P * 16)
    return fwd, bwd


def moe_kernel_work(cfg, n_active):
    """Algorithmic (flops, bytes) per launch of each kernel step (weights of
    the active experts only)."""
    P, T, E, H, I, b = cfg.T * cfg.k, cfg.T, cfg.E, cfg.H, cfg.I, cfg.b
    wgu, wd = moe_weight_bytes(cfg)
    nblk = 2 * I // b
    rops = nblk * 2 * b * b * 2
    npair = b * (b - 1) // 2
    return {
        "moe.route": (0, T * E * 4 + P * 4 * 5 + T * (P // T) * 4),
        "moe.worklist": (0, E * 8),
        # gate/up GEMM + per-expert rotation: weights, the gathered tokens
        # (each read once), h and act written
        "moe.gateup": (2 * P * H * 2 * I + 2 * P * 2 * I * b, n_active * (wgu + rops) + T * H * 2 + P * 2 * I * 2
                       + P * I * 2),
        "moe.down": (2 * P * I * H, n_active * wd + P * I * 2 + P * H * 2),
        "moe.combine": (0, P * H * 2 + T * H * 2 + P * 8),
        # dA = dO . W_d per pair, SwiGLU backward: weights, dy (once), h read,
        # dH written
        "moe.dA": (2 * P * H * I, n_active * wd + T * H * 2 + P * 2 * I * 2 * 2 + P * 4),
        "moe.dw_reduce": (0, P * 4 * 3),
        # S = dH^T H per block and the rotated dH (2 P 2I b each): dH and h
        # read, dz written
        "moe.dq": (4 * P * 2 * I * b, P * 2 * I * 2 * 3 + n_active * nblk * b * b * 6 + E * nblk * npair * 4),
        "moe.dX": (2 * P * 2 * I * H, n_active * wgu + P * 2 * I * 2 + P * H * 2),
        "moe.unpermute": (0, P * H * 2 + T * H * 2 + P * 4),
        "moe.router_bwd": (0, 2 * T * E * 4 + 2 * P * 4),
        "cayley": (2 * E * nblk * b ** 3, E * nblk * (npair * 2 + b * b * 4 + 2 * b * b * 2)),
    }


def moe_cpu_baseline(cfg, inp, seconds):
    """The oracle's forward and backward of whole experts (every routed row
    of each), as many as fit in about `seconds`."""
    from oracle import codec, moe as omoe

    idx, w = omoe.route(inp["logits"], cfg.k)
    rt = omoe.group(idx, cfg.E, cfg.chunk)
    rt.update(idx=idx, w=w)
    act = [int(e) for e in rt["active"]]
    X = codec.bf16_bits_to_f64(inp["x"])
    dy = codec.bf16_bits_to_f64(inp["dy"])
    wflat = w.reshape(-1)
    done, t0 = [], time.perf_counter()
    for e in act:  # the oracle's per-expert forward and backward, expert by expert
        pairs = rt["perm"][rt["offsets"][e]:rt["offsets"][e + 1]]
        Wgu, Wd, R = omoe.expert_weights(inp, e)
        omoe.expert_forward(X[pairs // cfg.k], Wgu, Wd, R, cfg.I)
        omoe.expert_backward(inp, e, pairs, X, dy, wflat)
        done.append(e)
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    rows = int(sum(rt["counts"][e] for e in done))
    H, I, b = cfg.H, cfg.I, cfg.b
    gemm = 2 * rows * H * 2 * I + 2 * rows * I * H
    fl = 2 * gemm + 6 * rows * 2 * I * b
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{cfg.name}: {len(done)} of {len(act)} active experts ({rows} routed rows), "
                      f"dequant + Cayley + fwd + bwd in fp64 numpy, {dt:.2f} s"}


def moe_inputs(cfg, cache):
    """Seeded inputs; a workload that differs from one already drawn only in
    its token count takes that one's weights and its first T token rows."""
    from oft_inputs import make_moe, moe_token_rows

    for other in cache.values():
        oc = other["cfg"]
        if (oc.E, oc.k, oc.H, oc.I, oc.g, oc.b, oc.w_fmt, oc.bias_std) == (cfg.E, cfg.k, cfg.H, cfg.I, cfg.g,
                                                                          cfg.b, cfg.w_fmt, cfg.bias_std) \
                and oc.T >= cfg.T:
            return moe_token_rows(other, cfg)
    inp = make_moe(cfg, seed=0)
    cache[cfg.name] = inp
    return inp


def run_moe(cfg, args, sha, headline, cache):
    import numpy as np
    import torch

    import orthogonal_fine_tuning_amd as oft

    inp = moe_inputs(cfg, cache)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    T, E, k, H, I, b = cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.b
    P = T * k
    # the frozen INT4 weights in the tiled storage (a one-time permutation at
    # load, like the quantisation itself) where its shape constraint holds
    tiled = args.storage == "auto" and cfg.w_fmt == "int4" and H % 256 == 0 and I % 256 == 0
    w_fmt = oft.OFT_W_FP4_E2M1 if cfg.w_fmt == "fp4" else oft.OFT_W_INT4_TILED if tiled else oft.OFT_W_INT4
    d = oft.moe_desc(T, E, k, H, I, cfg.g, b, cfg.chunk, 0, w_fmt=w_fmt)
    i32 = dict(dtype=torch.int32, device="cuda")
    rtt = dict(topk_idx=torch.empty((T, k), **i32), topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
               counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32), perm=torch.empty(P, **i32),
               inv_perm=torch.empty(P, **i32), active=torch.empty(E, **i32), n_active=torch.empty(4, **i32),
               chunk_of_expert=torch.empty(E, **i32))
    rt = oft.moe_routing(**rtt)
    nblk = E * cfg.nblk_e
    q = dev(inp["p"])
    Rf = torch.empty((E, cfg.nblk_e, b, b), dtype=torch.float32, device="cuda")
    Rops = torch.empty((E, cfg.nblk_e, 2, b, b), dtype=torch.int16, device="cuda")
    W = {n: dev(inp[n]) for n in ("wgu_codes", "wgu_scales", "wd_codes", "wd_scales")}
    W_rm = None
    if tiled:
        W_rm, W = W, {n: torch.empty_like(t) for n, t in W.items()}
        for c, sc, rows, cols in (("wgu_codes", "wgu_scales", 2 * I, H), ("wd_codes", "wd_scales", H, I)):
            oft.oft_pack_int4_tiled(E, rows, cols, cfg.g, W_rm[c], W_rm[sc], W[c], W[sc])
        torch.cuda.synchronize()
    x, lg, dy = dev(inp["x"]), dev(inp["logits"]), dev(inp["dy"])
    hs = torch.empty((P, 2 * I), dtype=torch.int16, device="cuda")
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    dx = torch.empty((T, H), dtype=torch.int16, device="cuda")
    dq = torch.empty((E, cfg.nblk_e, cfg.npair), dtype=torch.float32, device="cuda")
    dw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    nbf = oft.oft_moe_workspace_bytes(d, oft.OFT_PASS_FWD)
    nbb = oft.oft_moe_workspace_bytes(d, oft.OFT_PASS_BWD)
    wsf = torch.empty(nbf, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(nbb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def fwd():
        oft.oft_moe_grouped_fwd(d, x, lg, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"], Rops, rt,
                                hs, y, wsf, nbf, stream=sp)

    def bwd():
        oft.oft_moe_grouped_bwd(d, dy, rt, hs, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"], Rf,
                                Rops, dx, dq, dw, wsb, nbb, stream=sp)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        oft.cayley_build(q, nblk, b, Rf, Rops, stream=sp)
        if ev is not None:
            ev[1].record(stream)
        fwd()
        if ev is not None:
            ev[2].record(stream)
        bwd()
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    t_step, (t_cay, t_fwd, t_bwd) = time_steps(step, args.steps, 0)
    transient = torch.cuda.max_memory_allocated() - mem0  # the library allocates nothing
    n_active = int(rtt["n_active"][0].item())
    kern = profile_steps(step, args.prof_steps)
    f_fwd, f_bwd = moe_flops(cfg)
    by_fwd, by_bwd = moe_bytes(cfg, n_active)
    out = summary(cfg.name, t_step, f_fwd + f_bwd, by_fwd + by_bwd, kern, moe_kernel_work(cfg, n_active), sha,
                  {"cayley_build": t_cay, "fwd": t_fwd, "bwd": t_bwd})
    out["config"] = {"workload": cfg.name, "tokens": T, "experts": E, "top_k": k, "hidden": H,
                     "expert_intermediate": I, "weights": f"{cfg.w_fmt}_g{cfg.g}", "oft_block": b,
                     "weight_storage": "tiled" if tiled else "row-major",
                     "chunk": cfg.chunk, "active_experts": n_active, "parallelism": "single_gpu"}
    out["phase_rates"] = {"fwd_tflops": round(f_fwd / t_fwd / 1e12, 2), "bwd_tflops": round(f_bwd / t_bwd / 1e12, 2),
                          "fwd_alg_gbs": round(by_fwd / t_fwd / 1e9, 1), "bwd_alg_gbs": round(by_bwd / t_bwd / 1e9, 1)}
    out["transient_bytes"] = int(transient)
    if W_rm is not None:
        # the same step on the row-major storage of the same weights
        d_rm = oft.moe_desc(T, E, k, H, I, cfg.g, b, cfg.chunk, 0, w_fmt=oft.OFT_W_INT4)
        nbf_rm = oft.oft_moe_workspace_bytes(d_rm, oft.OFT_PASS_FWD)
        nbb_rm = oft.oft_moe_workspace_bytes(d_rm, oft.OFT_PASS_BWD)
        wsf_rm = torch.empty(nbf_rm, dtype=torch.uint8, device="cuda")
        wsb_rm = torch.empty(nbb_rm, dtype=torch.uint8, device="cuda")

        def step_rm(ev=None):
            if ev is not None:
                ev[0].record(stream)
            oft.cayley_build(q, nblk, b, Rf, Rops, stream=sp)
            oft.oft_moe_grouped_fwd(d_rm, x, lg, W_rm["wgu_codes"], W_rm["wgu_scales"], W_rm["wd_codes"],
                                    W_rm["wd_scales"], Rops, rt, hs, y, wsf_rm, nbf_rm, stream=sp)
            oft.oft_moe_grouped_bwd(d_rm, dy, rt, hs, W_rm["wgu_codes"], W_rm["wgu_scales"], W_rm["wd_codes"],
                                    W_rm["wd_scales"], Rf, Rops, dx, dq, dw, wsb_rm, nbb_rm, stream=sp)
            if ev is not None:
                ev[1].record(stream)

        t_rm, _ = time_steps(step_rm, args.steps, args.warmup, nev=2)
        out["row_major_storage"] = {"ms_per_step": round(t_rm * 1e3, 4),
                                    "speedup_of_tiled": round(t_rm / t_step, 4)}
        del wsf_rm, wsb_rm
    if not args.no_extras:
        dl = torch.empty((T, E), dtype=torch.float32, device="cuda")
        t_rb = burst_seconds(stream, lambda: oft.oft_moe_router_bwd(d, lg, rtt["topk_idx"], dw, dl, stream=sp))
        out["router_bwd"] = roofline(*moe_kernel_work(cfg, n_active)["moe.router_bwd"], t_rb)
        del dl
        # reference-policy forward: the frozen base alone (no rotation, no saved activations)
        t_base = burst_seconds(stream, lambda: oft.oft_moe_grouped_fwd_base(
            d, x, lg, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"], rt, None, y, wsf, nbf,
            stream=sp), 3)
        rops_bytes = n_active * cfg.nblk_e * 2 * b * b * 2
        out["reference_policy_fwd"] = roofline(2 * P * H * 2 * I + 2 * P * I * H,
                                               by_fwd - rops_bytes - P * 2 * I * 2, t_base)
    if not args.no_cold:
        cf, cb = cold_phases(fwd, bwd)
        out["phases_cold_us"] = {"fwd": round(cf * 1e6, 2), "bwd": round(cb * 1e6, 2),
                                 "fwd_alg_gbs": round(by_fwd / cf / 1e9, 1), "bwd_alg_gbs": round(by_bwd / cb / 1e9, 1)}
    if not args.no_dense_ref:
        del W, W_rm
        torch.cuda.empty_cache()
        out["dense_bf16_reference"] = moe_dense_reference(cfg, inp, args, dict(
            x=x, lg=lg, dy=dy, rt=rt, Rf=Rf, Rops=Rops, hs=hs, y=y, dx=dx, dq=dq, dw=dw, counts=rtt["counts"]),
            t_fwd + t_bwd)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = moe_cpu_baseline(cfg, inp, args.cpu_seconds * (3 if headline else 1))
    return out


def moe_dense_reference(cfg, inp, args, bufs, t_ours):
    """The same grouped kernels with every expert's weights dequantised to
    bf16 in HBM beforehand (not timed): the dense-weight reference of the
    fwd + bwd calls.  Same routing, inputs, outputs and step count."""
    import numpy as np
    import torch

    import orthogonal_fine_tuning_amd as oft

    T, E, k, H, I, b, g = cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.b, cfg.g
    d16 = oft.moe_desc(T, E, k, H, I, g, b, cfg.chunk, 0, w_fmt=oft.OFT_W_BF16)
    wgu = torch.empty((E, 2 * I, H), dtype=torch.int16, device="cuda")
    wd = torch.empty((E, H, I), dtype=torch.int16, device="cuda")
    for name, rows, cols, out in (("wgu", E * 2 * I, H, wgu), ("wd", E * H, I, wd)):
        codes = torch.from_numpy(np.ascontiguousarray(inp[f"{name}_codes"])).to("cuda")
        scales = torch.from_numpy(np.ascontiguousarray(inp[f"{name}_scales"]).view(np.int16)).to("cuda")
        oft.oft_dequant(oft.OFT_W_FP4_E2M1 if cfg.w_fmt == "fp4" else oft.OFT_W_INT4, rows, cols, g, codes,
                        scales, out)
        del codes, scales
    nbf = oft.oft_moe_workspace_bytes(d16, oft.OFT_PASS_FWD)
    nbb = oft.oft_moe_workspace_bytes(d16, oft.OFT_PASS_BWD)
    wsf = torch.empty(nbf, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(nbb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    B = bufs

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        oft.oft_moe_grouped_fwd(d16, B["x"], B["lg"], wgu, None, wd, None, B["Rops"], B["rt"], B["hs"], B["y"],
                                wsf, nbf, stream=sp)
        if ev is not None:
            ev[1].record(stream)
        oft.oft_moe_grouped_bwd(d16, B["dy"], B["rt"], B["hs"], wgu, None, wd, None, B["Rf"], B["Rops"], B["dx"],
                                B["dq"], B["dw"], wsb, nbb, stream=sp)
        if ev is not None:
            ev[2].record(stream)

    _, (t_fwd, t_bwd) = time_steps(step, args.steps, args.warmup, nev=3)
    del wsf, wsb
    lib_ref = {"fwd_us": round(t_fwd * 1e6, 2), "bwd_us": round(t_bwd * 1e6, 2),
               "weights_bytes": int(E * 3 * I * H * 2),
               "ratio": round(t_ours / (t_fwd + t_bwd), 4),
               "note": "fwd+bwd time of the 4-bit path over that of the same kernels on bf16 weights"}
    lib_ref["torch_per_expert"] = moe_torch_reference(cfg, wgu, wd, bufs["counts"], t_ours)
    del wgu, wd
    torch.cuda.empty_cache()
    return lib_ref


def moe_torch_reference(cfg, wgu, wd, counts, t_ours, reps=5):
    """The grouped GEMMs as torch bf16 matrix products (hipBLASLt), one per
    active expert on the same routing (counts: the routed rows of each
    expert): forward gate/up and down, backward dA (dO W_down) and dX
    (dH W_gu), on random bf16 rows of the same shapes; captured once in a
    HIP graph and replayed, so that no product waits for the host.  The
    4-bit path's rotation, SwiGLU, dQ, routing and combine have no
    counterpart here, so its time is compared with more work."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    H, I = cfg.H, cfg.I
    cnt = counts.cpu().numpy().astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(cnt)])
    P = int(offs[-1])
    bf = dict(dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(0)
    xs = torch.randn(P, H, generator=gen, **bf)
    act = torch.randn(P, I, generator=gen, **bf)
    dO = torch.randn(P, H, generator=gen, **bf)
    dH = torch.randn(P, 2 * I, generator=gen, **bf)
    Wgu = wgu.view(torch.bfloat16)  # [E, 2I, H]
    Wd = wd.view(torch.bfloat16)    # [E, H, I]
    active = [e for e in range(cfg.E) if cnt[e] > 0]
    keep = []

    def fwd():
        for e in active:
            a, b = int(offs[e]), int(offs[e + 1])
            keep.append(F.linear(xs[a:b], Wgu[e]))   # [n, 2I]
            keep.append(F.linear(act[a:b], Wd[e]))   # [n, H]

    def bwd():
        for e in active:
            a, b = int(offs[e]), int(offs[e + 1])
            keep.append(torch.mm(dO[a:b], Wd[e]))    # [n, I]
            keep.append(torch.mm(dH[a:b], Wgu[e]))   # [n, H]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture (library handles, workspaces)
        fwd()
        bwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    keep.clear()
    graphs = []
    for f in (fwd, bwd):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    torch.cuda.synchronize()
    ts = []
    for g in graphs:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        g.replay()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        ts.append(ev[0].elapsed_time(ev[1]) * 1e-3 / reps)
    del graphs, keep, xs, act, dO, dH
    torch.cuda.empty_cache()
    flops = 2 * 2 * P * H * 2 * I + 2 * 2 * P * I * H
    return {"fwd_us": round(ts[0] * 1e6, 2), "bwd_us": round(ts[1] * 1e6, 2),
            "tflops": round(flops / (ts[0] + ts[1]) / 1e12, 1), "experts": len(active),
            "ratio": round(t_ours / (ts[0] + ts[1]), 4),
            "note": "fwd+bwd time of the 4-bit path over torch bf16 per-expert GEMMs (gate/up, down, dA, dX) "
                    "on the same routing, replayed from a HIP graph"}


# ------------------------------------------------------------------ counter summaries
PMC_PASSES = {
    # one rocprofv3 --pmc run each (at most 8 SQ and 4 TCC counters per run)
    "sq": "GRBM_GUI_ACTIVE SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
          "SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU SQ_INSTS_MFMA",
    "wait": "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS "
            "SQ_INSTS_LDS SQ_INSTS_SALU",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
PMC_BENCH = ("python3 bench.py --config {w} --steps 2 --warmup 1 --prof-steps 1 --no-cold --no-extras "
             "--no-dense-ref --no-cpu-baseline --calibrate-copy-mib {mib}")
TRACE_BENCH = ("python3 bench.py --config {w} --steps 5 --warmup 1 --prof-steps 1 --no-cold --no-extras "
               "--no-dense-ref --no-cpu-baseline")
CLOCK_GHZ = 2.4  # nominal shader clock for the VALU-busy estimate


def kernel_region(name):
    """The library step (bench.py kernel-table name) a kernel belongs to, from
    its name and template arguments; None for kernels outside the library."""
    base = re.sub(r"^(void )?oft::(\(anonymous namespace\)::)?", "", name)
    fam, _, targs = base.partition("<")
    a = [t.strip() for t in targs.rstrip(">").split(",")] if targs else []
    nt = {"gemm_nt_dma_kernel": (3, 5), "gemm_nt_dec4_kernel": (1, 2), "gemm_nt_dec_kernel": (2, 3),
          "gemm_nt_kernel": (4, 5), "gemm_nt_dec16_kernel": (1, None), "gemm_nt_skinny_kernel": (5, None),
          "gemm_nt_hl_kernel": (2, 3)}
    nn = {"gemm_nn_kernel": (5, 6), "gemm_nn_dma_kernel": (1, 2), "gemm_nn_q4_kernel": (0, 1)}
    if fam in nt:
        ie, ig = nt[fam]
        epi = int(a[ie]) if len(a) > ie else 0
        grouped = ig is not None and len(a) > ig and a[ig] == "true"
        if grouped:
            return "moe.down" if epi == 1 else "moe.gateup"
        return {0: "dense.fwd", 1: "dense.dx", 3: "dense.fwd_base"}.get(epi, "dense.fwd")
    if fam in nn:
        ie, ig = nn[fam]
        epi = int(a[ie]) if len(a) > ie else 0
        grouped = len(a) > ig and a[ig] == "true"
        if grouped:
            return "moe.dA" if epi == 1 else "moe.dX"
        return "dense.dx"
    for pre, reg in (("dq_dma", "dense.dq"), ("dq_partial", "dense.dq"), ("dq_final", "dense.dq_final"),
                     ("split_reduce", "dense.dx_reduce"), ("transpose_", "dense.transpose"), ("cayley", "cayley"),
                     ("slots_latch", "dense.slots_latch"), ("moe_dq", "moe.dq"), ("moe_combine", "moe.combine"),
                     ("moe_unpermute", "moe.unpermute"), ("moe_worklist", "moe.worklist"),
                     ("moe_dw_reduce", "moe.dw_reduce"), ("moe_router_bwd", "moe.router_bwd"),
                     ("moe_", "moe.route"), ("logprob", "policy.logprob_diff")):
        if fam.startswith(pre):
            return reg
    return None


def _read_dispatches(path):
    """rocprofv3 counter CSV -> [{name, dur_us, counter: value}] in dispatch order."""
    disp = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = disp.setdefault(r["Dispatch_Id"], {"name": re.sub(r"\((?!anonymous).*$", "", r["Kernel_Name"])})
            d["dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp, key=int)]


def _mean_by_kernel(dispatches):
    acc = {}
    for d in dispatches:
        e = acc.setdefault(d["name"], {"n": 0})
        e["n"] += 1
        for k, v in d.items():
            if k != "name":
                e[k] = e.get(k, 0.0) + v
    return {n: {k: (v / e["n"] if k != "n" else v) for k, v in e.items()} for n, e in acc.items()}


def pmc_summary(root, copy_mib=256):
    """Write profiles/traffic.json and profiles/pmc_<workload>.md (and
    profiles/kernels_<workload>.md from a kernel trace) from rocprofv3 runs
    laid out as root/<workload>/<pass>/run_counter_collection.csv (passes of
    PMC_PASSES) and root/<workload>/trace/run_kernel_stats.csv; each pass's
    benchmark line in root/<workload>/<pass>.json.  HBM bytes: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what they read for the plain
    copy of copy_mib MiB run in the same process (the copy dispatch that
    wrote the most)."""
    prof = os.path.join(ROOT, "profiles")
    entries, calib, shas = {}, {}, set()
    cmds = [f"rocprofv3 --pmc {c} -d {root}/{{w}}/{p} -o run --output-format csv -- "
            + PMC_BENCH.format(w="{w}", mib=copy_mib) for p, c in PMC_PASSES.items()]
    cmds.append(f"rocprofv3 --kernel-trace --stats -d {root}/{{w}}/trace -o run --output-format csv -- "
                + TRACE_BENCH.format(w="{w}"))
    for w in sorted(os.listdir(root)):
        wdir = os.path.join(root, w)
        if not os.path.isdir(wdir):
            continue
        per = {}
        for p in PMC_PASSES:
            f = os.path.join(wdir, p, "run_counter_collection.csv")
            if os.path.exists(f):
                per[p] = _read_dispatches(f)
            j = os.path.join(wdir, p + ".json")
            if os.path.exists(j):
                with open(j) as fh:
                    for line in fh:
                        if line.startswith("{"):
                            shas.add(json.loads(line)["roofline"].get("source_sha"))
        factors = {}
        for p, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
            copies = [d for d in per.get(p, []) if "copyBuffer" in d["name"] and ctr in d]
            if copies:
                c = max(copies, key=lambda d: d[ctr])
                factors[p] = copy_mib * 1024.0 / c[ctr] if c[ctr] > 0 else None
        calib[w] = {"copy_mib": copy_mib, "fetch_factor": factors.get("fetch"), "write_factor": factors.get("write")}
        means = {p: _mean_by_kernel([d for d in ds if kernel_region(d["name"])]) for p, ds in per.items()}
        names = set()
        for m in means.values():
            names |= set(m)
        rows = []
        for n in names:
            sq, wt = means.get("sq", {}).get(n, {}), means.get("wait", {}).get(n, {})
            fe, wr = means.get("fetch", {}).get(n, {}), means.get("write", {}).get(n, {})
            dur = sq.get("dur_us") or wt.get("dur_us") or fe.get("dur_us") or 0.0
            calls = max(e.get("n", 0) for e in (sq, wt, fe, wr))
            r = {"kernel": n.replace("void ", ""), "region": kernel_region(n), "dur_us": dur, "calls": calls}
            if sq and dur > 0:
                r["mfma_pct"] = 100.0 * sq.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) * 1024 / (dur * 1e-6) / (PEAK_BF16_TFLOPS * 1e12)
                r["valu_pct"] = 100.0 * sq.get("SQ_ACTIVE_INST_VALU", 0) * 4 / (1024 * dur * 1e3 * CLOCK_GHZ)
                mf = sq.get("SQ_INSTS_MFMA", 0)
                r["valu_per_mfma"] = sq.get("SQ_INSTS_VALU", 0) / mf if mf else None
                lds = sq.get("SQ_ACTIVE_INST_LDS", 0)
                r["lds_conflict_pct"] = 100.0 * sq.get("SQ_LDS_BANK_CONFLICT", 0) / lds if lds else None
            if wt and wt.get("SQ_WAVE_CYCLES"):
                wc = wt["SQ_WAVE_CYCLES"]
                r["wait_pct"] = 100.0 * wt.get("SQ_WAIT_ANY", 0) / wc
                r["issue_wait_pct"] = 100.0 * wt.get("SQ_WAIT_INST_ANY", 0) / wc
                r["active_pct"] = 100.0 * wt.get("SQ_ACTIVE_INST_ANY", 0) / wc
            if fe and factors.get("fetch"):
                r["fetch_mb"] = fe.get("FETCH_SIZE", 0) * factors["fetch"] * 1024 / 1e6
            if wr and factors.get("write"):
                r["write_mb"] = wr.get("WRITE_SIZE", 0) * factors["write"] * 1024 / 1e6
            rows.append(r)
        rows.sort(key=lambda r: -r["dur_us"] * r["calls"])
        # traffic of each library step: its kernel with the most time (one launch per step)
        seen = set()
        for r in rows:
            if r["region"] in seen or "fetch_mb" not in r or "write_mb" not in r:
                continue
            seen.add(r["region"])
            entries[f"{r['region']}:{w}"] = {
                "kernel": r["kernel"], "fetch_bytes": round(r["fetch_mb"] * 1e6),
                "write_bytes": round(r["write_mb"] * 1e6),
                "bytes_per_launch": round((r["fetch_mb"] + r["write_mb"]) * 1e6)}

        def fmt(v, d=1):
            return "—" if v is None else f"{v:.{d}f}"
        total = sum(r["dur_us"] * r["calls"] for r in rows) or 1.0
        lines = [f"# rocprofv3 counters: `{w}` (Cayley build + forward + backward, one GPU)", "",
                 "Commands (from the repository root on the MI355X box, `cd /tmp && export TMPDIR=/tmp` first; "
                 "one run per counter set):", "", "```"]
        lines += [c.format(w=w) for c in cmds]
        lines += [f"python3 bench.py --pmc-summary {root}", "```", "",
                  "Per kernel, averaged over its dispatches in the counter runs (which also cover the warm-up "
                  "and the profiled step).  MFMA % = matrix-core busy cycles x 1024 flop per cycle per SIMD "
                  "over the kernel's duration, against the 2.5 PFLOP/s bf16 peak (padding rows included).  "
                  f"VALU % = VALU instruction cycles (4 per instruction) over 1024 SIMDs x duration at "
                  f"{CLOCK_GHZ} GHz.  LDS conflict % = bank-conflict cycles over LDS-active cycles.  Wait / "
                  "issue-wait / active = SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_ANY over wave-cycles.  "
                  "Fetch / write: FETCH_SIZE, WRITE_SIZE per dispatch, scaled by "
                  f"{fmt(factors.get('fetch'), 3)} / {fmt(factors.get('write'), 3)} (a plain {copy_mib} MiB "
                  "device copy in the same process).", "",
                  "| step | kernel | calls | µs | share | MFMA % | VALU % | VALU/MFMA | LDS conflict % | wait % | "
                  "issue-wait % | active % | fetch MB | write MB |",
                  "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for r in rows[:14]:
            lines.append(
                f"| {r['region']} | `{r['kernel']}` | {r['calls']} | {r['dur_us']:.2f} | "
                f"{100 * r['dur_us'] * r['calls'] / total:.1f}% | {fmt(r.get('mfma_pct'))} | {fmt(r.get('valu_pct'))} | "
                f"{fmt(r.get('valu_per_mfma'))} | {fmt(r.get('lds_conflict_pct'))} | {fmt(r.get('wait_pct'))} | "
                f"{fmt(r.get('issue_wait_pct'))} | {fmt(r.get('active_pct'))} | {fmt(r.get('fetch_mb'), 2)} | "
                f"{fmt(r.get('write_mb'), 2)} |")
        with open(os.path.join(prof, f"pmc_{w}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        # kernel trace
        st = os.path.join(wdir, "trace", "run_kernel_stats.csv")
        if os.path.exists(st):
            with open(st) as f:
                recs = [r for r in csv.DictReader(f)]
            recs = [r for r in recs if kernel_region(re.sub(r"\((?!anonymous).*$", "", r["Name"]))]
            tot = sum(float(r["TotalDurationNs"]) for r in recs) or 1.0
            recs.sort(key=lambda r: -float(r["TotalDurationNs"]))
            tl = [f"# rocprofv3 kernel trace: `{w}` (5 timed steps, 1 warm-up, 1 profiled)", "", "Command (from "
                  "the repository root on the MI355X box, `cd /tmp && export TMPDIR=/tmp` first):", "", "```",
                  cmds[-1].format(w=w), f"python3 bench.py --pmc-summary {root}", "```", "",
                  "Library kernels only (torch's fill and spin kernels and the host copies left out); share of "
                  "their summed time.", "", "| step | kernel | calls | avg µs | min µs | max µs | share |",
                  "|---|---|---:|---:|---:|---:|---:|"]
            for r in recs[:16]:
                nm = re.sub(r"\((?!anonymous).*$", "", r["Name"]).replace("void ", "")
                tl.append(f"| {kernel_region(nm)} | `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                          f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                          f"{100 * float(r['TotalDurationNs']) / tot:.1f}% |")
            with open(os.path.join(prof, f"kernels_{w}.md"), "w") as f:
                f.write("\n".join(tl) + "\n")
    shas.discard(None)
    out = {"_about": "HBM bytes per launch of each library step's main kernel, from rocprofv3 FETCH_SIZE and "
                     "WRITE_SIZE runs of bench.py per workload, scaled by the same counters on a plain device "
                     "copy in the same process; bench.py reports them only while source_sha matches the "
                     "kernel sources.",
           "source_sha": shas.pop() if len(shas) == 1 else source_sha(),
           "commands": [c for c in cmds] + [f"python3 bench.py --pmc-summary {root}"],
           "copy_calibration": calib, "entries": entries}
    with open(os.path.join(prof, "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


# ------------------------------------------------------------------ targets
DECODE_SHAPES = ("gateup_4b_decode", "moe_1t_decode")


def targets(name, r):
    """The step's share of its roofline against the target for its class
    (at least 60 % at large token counts, 70 % of HBM on the decode shapes),
    and for MoE the fwd + bwd time over the dense bf16 references (at most
    1.2); 'gap' is target over achieved (above 1: short of the target)."""
    if name == "tiny_qkv":
        return {"note": "parity-sized shape; no target"}
    sr = r["step_roofline"]
    want = 0.7 if name in DECODE_SHAPES else 0.6
    out = {"step_roofline_frac": {"bound": sr["bound"], "target": want, "achieved": sr["frac"],
                                  "gap": round(want / sr["frac"], 2) if sr["frac"] > 0 else None}}
    ref = r.get("dense_bf16_reference")
    if ref:
        out["moe_over_dense_bf16_same_kernels"] = {"target_max": 1.2, "achieved": ref["ratio"]}
        tp = ref.get("torch_per_expert")
        if tp:
            out["moe_over_torch_bf16_per_expert"] = {"target_max": 1.2, "achieved": tp["ratio"]}
    return out


# ------------------------------------------------------------------ summary
def summary(name, t_step, flops, nbytes, kern, work, sha, phases):
    """The step's rate and roofline, the kernel-step table and the dominant
    kernel step's roofline."""
    kernels = {}
    for kname, (ms, calls) in sorted(kern.items(), key=lambda kv: -kv[1][0]):
        ent = {"us_per_step": round(ms * 1e3, 2), "launches_per_step": round(calls, 2)}
        if kname in work and calls > 0:
            f, by = work[kname]
            per = ms * 1e-3 / calls
            r = roofline(f, by, per)
            ent.update(bound=r["bound"], achieved=r["achieved"], unit=r["unit"], frac=r["frac"])
        kernels[kname] = ent
    dom = max(kern, key=lambda kk: kern[kk][0])
    ms, calls = kern[dom]
    f, by = work.get(dom, (0, 0))
    roof = roofline(f, by, ms * 1e-3 / max(calls, 1), kernel=dom, traffic=load_traffic(f"{dom}:{name}", sha))
    roof["timing"] = ("HIP events the library records on the launch stream around this step of its work, "
                      "averaged over profiled steps right after the timed steps")
    roof["source_sha"] = sha
    return {
        "value": round(flops / t_step / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(t_step * 1e3, 4),
        "roofline": roof,
        "step_roofline": roofline(flops, nbytes, t_step),
        "phases_us": {k: round(v * 1e6, 2) for k, v in phases.items()},
        "kernels": kernels,
    }


def main():
    args = parse()
    if args.pmc_summary is not None:
        pmc_summary(args.pmc_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; --gpus must be 1 "
                                   "(sharding over several GPUs is designed, not implemented)"}))
        sys.exit(2)

    import torch

    import orthogonal_fine_tuning_amd as oft
    from oft_inputs import CONFIGS

    oft._lib.load()
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = ORDER if args.config == "all" else [args.config]
    head = HEADLINE if args.config == "all" else args.config
    sha = source_sha()
    cache = {}
    results = {}
    for name in names:
        cfg = CONFIGS[name]
        if args.w_fmt is not None and cfg.w_fmt in ("int4", "fp4"):
            cfg = cfg.with_(w_fmt=args.w_fmt)
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        if hasattr(cfg, "segs"):
            results[name] = run_dense(cfg, args, sha, name == head)
        else:
            results[name] = run_moe(cfg, args, sha, name == head, cache)
        results[name]["bench_seconds"] = round(time.perf_counter() - t0, 1)
        results[name]["targets"] = targets(name, results[name])
        if name == "moe_1t_decode" or len(names) == 1:
            cache.clear()
    h = results[head]
    line = {"metric": METRIC, "value": h["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": h["config"],
            "roofline": h["roofline"]}
    if "cpu_baseline" in h:
        line["cpu_baseline"] = h["cpu_baseline"]
    for k, v in h.items():
        if k not in line and k != "value":
            line[k] = v
    if len(names) > 1:
        line["workloads"] = {n: r for n, r in results.items() if n != head}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
