#!/usr/bin/env python3
"""Benchmark of the OFT dequant-GEMM hot path on one MI355X.

One step = one pass of the whole dense path over one batch: Cayley build of
the adapter rotations, the forward (dequant GEMM + split-projection rotation
epilogue) and the backward (dX with the rotation prologue, and dQ).  The
default workload is the fused Q/K/V projection of a 4B-shaped model: 4096
tokens, hidden 2560, out 6144 = 4096 + 1024 + 1024, FP8 e4m3 weights with
per-channel scales, OFT blocks of 32.  Inputs are seeded synthetic data,
resident in HBM before timing starts.

Prints ONE JSON line (rank 0).  ``value`` is algorithmic TFLOP/s of the
whole step (fwd 2MNK + 2MNb, bwd 2MNK + 4MNb; the Cayley build is timed but
its flops are not counted).  ``roofline`` reports the forward GEMM kernel:
algorithmic flops per launch over its mean duration against the bf16
matrix peak, or, for shapes below the ridge point (312.5 flop per byte:
the weight streams of few-token layers), algorithmic bytes per launch
against HBM; the duration comes from HIP events on the launch stream
around a burst of back-to-back forward launches right after the timed
steps, queued behind a short GPU spin so that the host's cost per call
leaves no gaps (``phases_us`` comes from events around each phase of every
timed step and also counts the idle time an event boundary adds).
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.  MoE workloads also report ``transient_bytes`` (peak device memory
allocated during the timed calls beyond what existed before them) and
``dense_bf16_reference``: the same fwd + bwd calls on every expert's weights
dequantised to bf16 beforehand (``--no-dense-ref`` skips it), with the ratio
of the INT4 path's time to it.  Dense workloads also report
``reference_policy_fwd``: the frozen base alone (``oft_linear_fwd_base``, the
KL reference), and ``slots_fwd`` (``oft_linear_fwd_slots``: the forward on
the active slot of a double-buffered adapter, latch launch included), timed
the same way as ``roofline``; MoE workloads report
``router_bwd`` (``oft_moe_router_bwd``: d_logits from the combine-weight
gradient, outside the step) the same way.  ``phases_cold_us`` times
fwd and bwd again, each right after evicting the last-level cache, so that
the weights stream from HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "OFT dequant-GEMM fwd+bwd TFLOP/s and HBM GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte where the two meet (312.5)


def roofline_object(mfma_bound, flops, nbytes, seconds, kernel, traffic):
    """Above the ridge point: algorithmic TFLOP/s against the bf16 matrix
    peak; below it (the weight streams of few-token shapes): algorithmic
    GB/s against HBM."""
    if mfma_bound:
        achieved, peak, unit = flops / seconds / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / seconds / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"bound": "mfma" if mfma_bound else "hbm", "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel,
            "kernel_us": round(seconds * 1e6, 2), "algorithmic_flops": int(flops), "algorithmic_bytes": int(nbytes)}


def burst_seconds(stream, launch, n=10):
    """Mean duration of one of n back-to-back launches: HIP events on the
    launch stream around the burst.  A short GPU spin is queued first, so
    every launch is already in the queue when the first event fires and the
    host's cost per call adds no idle time between the kernels."""
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="qkv_4b")
    ap.add_argument("--w-fmt", choices=("int4", "fp4"), default=None,
                    help="run a 4-bit workload with this base format (FP4: OCP MX E2M1 codes, E8M0 group "
                         "exponents in the same layout and bytes as INT4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-ref", action="store_true",
                    help="MoE: skip the dense-bf16-weight reference run of the same grouped kernels")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip phases_cold_us (keeps a profiler's kernel averages to the timed steps)")
    ap.add_argument("--cpu-rows", type=int, default=1 << 30,
                    help="token rows of the oracle sample for cpu_baseline")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (a reference "
                         "for HBM byte counters)")
    return ap.parse_args()


def dense_flops(cfg):
    M, N, K, b = cfg.M, cfg.N, cfg.K, cfg.b
    fwd = 2 * M * N * K + 2 * M * N * b
    bwd = 2 * M * N * K + 4 * M * N * b
    return fwd, bwd


def dense_bytes(cfg):
    """Algorithmic HBM bytes: what the method must read and write once."""
    M, N, K, b = cfg.M, cfg.N, cfg.K, cfg.b
    xb = 4 if cfg.x_dtype == "f32" else 2
    if cfg.w_fmt in ("int4", "fp4"):
        wbytes = N * K // 2 + N * (K // cfg.g) * 2
    else:
        wbytes = N * K + N * 4
    nblk = N // b
    rops = nblk * 2 * b * b * 2
    rf = nblk * b * b * 4
    npair = b * (b - 1) // 2
    fwd = wbytes + M * K * xb + M * N * xb + rops
    bwd = wbytes + M * N * 2 + M * N * xb + M * K * xb + rops + rf + nblk * npair * 4
    return fwd, bwd


FWD_KERNEL_SOURCES = ["orthogonal_fine_tuning_amd/csrc/linear_fwd.hip",
                      "orthogonal_fine_tuning_amd/csrc/gemm_nt.h",
                      "orthogonal_fine_tuning_amd/csrc/gemm_nt_dma.h",
                      "orthogonal_fine_tuning_amd/csrc/gemm_skinny.h",
                      "orthogonal_fine_tuning_amd/csrc/oft_device.h",
                      "orthogonal_fine_tuning_amd/csrc/oft_formats.h"]


def fwd_kernel_name(cfg):
    """The kernel oft_linear_fwd launches for this shape (one launch per call)."""
    if cfg.x_dtype == "bf16":
        if cfg.M <= 64:
            return "gemm_nt_dec4_kernel" if cfg.w_fmt != "fp8" and cfg.K % 256 == 0 else "gemm_nt_dec_kernel"
        return "gemm_nt_dma_kernel"
    if cfg.M <= 64 and cfg.K % 256 == 0:
        return "gemm_nt_skinny_kernel"
    return "gemm_nt_kernel"


def kernel_source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, sha):
    """HBM traffic per launch from committed rocprofv3 counter runs, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_sha") != sha:
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(cfg, inp, rows):
    import numpy as np
    from oracle import dense as odense

    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - informational only
        cores = os.cpu_count() or 1
    ms = min(rows, cfg.M)
    sub = dict(inp)
    sub["cfg"] = cfg.with_(M=ms)
    sub["x"] = inp["x"][:ms]
    sub["dy"] = inp["dy"][:ms]
    reps, t0 = 0, time.perf_counter()
    while True:  # repeat the sample for at least ~10 s of CPU work
        odense.run(sub)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 50:
            break
    f, b = dense_flops(sub["cfg"])
    return {"value": reps * (f + b) / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{cfg.name}: {ms} of {cfg.M} token rows, dequant + Cayley + fwd + bwd (dX, dQ) "
                      f"in fp64 numpy, {reps} repetitions in {dt:.1f} s"}


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


def moe_flops(cfg):
    P, H, I, b = cfg.T * cfg.k, cfg.H, cfg.I, cfg.b
    gemm = 2 * P * H * 2 * I + 2 * P * I * H
    return gemm + 2 * P * 2 * I * b, gemm + 4 * P * 2 * I * b


def moe_bytes(cfg, n_active):
    P, T, E, H, I, g, b = cfg.T * cfg.k, cfg.T, cfg.E, cfg.H, cfg.I, cfg.g, cfg.b
    w_e = 2 * I * H // 2 + 2 * I * (H // g) * 2 + H * I // 2 + H * (I // g) * 2
    nblk = 2 * I // b
    rops = nblk * 2 * b * b * 2
    fwd = n_active * (w_e + rops) + T * H * 2 + T * E * 4 + P * 2 * I * 2 + T * H * 2 + P * 16
    bwd = (n_active * (w_e + rops + nblk * b * b * 4) + T * H * 2 + P * 2 * I * 2 + T * H * 2
           + E * nblk * (b * (b - 1) // 2) * 4 + P * 4 + P * 16)
    return fwd, bwd


def run_moe(cfg, args):
    import numpy as np
    import torch

    import orthogonal_fine_tuning_amd as oft
    from oft_inputs import make_moe

    inp = make_moe(cfg, seed=0)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to("cuda")

    T, E, k, H, I, b = cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.b
    P = T * k
    d = oft.moe_desc(T, E, k, H, I, cfg.g, b, cfg.chunk, 0,
                     w_fmt=oft.OFT_W_FP4_E2M1 if cfg.w_fmt == "fp4" else oft.OFT_W_INT4)
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

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        oft.cayley_build(q, nblk, b, Rf, Rops, stream=sp)
        if ev is not None:
            ev[1].record(stream)
        oft.oft_moe_grouped_fwd(d, x, lg, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"], Rops, rt,
                                hs, y, wsf, nbf, stream=sp)
        if ev is not None:
            ev[2].record(stream)
        oft.oft_moe_grouped_bwd(d, dy, rt, hs, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"], Rf,
                                Rops, dx, dq, dw, wsb, nbb, stream=sp)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    mem0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    transient = torch.cuda.max_memory_allocated() - mem0  # the library allocates nothing
    n_active = int(rtt["n_active"][0].item())
    # the router backward (d_logits from dw through the softmax top-k), not
    # part of the step: a burst of launches on the step's routing and dw
    dl = torch.empty((T, E), dtype=torch.float32, device="cuda")
    burst = 10
    t_rb = burst_seconds(stream, lambda: oft.oft_moe_router_bwd(d, lg, rtt["topk_idx"], dw, dl, stream=sp), burst)
    by_rb = 2 * T * E * 4 + 2 * T * k * 4  # logits in, d_logits out, idx and dw in
    rb_roof = roofline_object(False, 0, by_rb, t_rb, kernel="moe_router_bwd_kernel", traffic=None)
    rb_roof["kernel_timing"] = (f"HIP events around {burst} back-to-back launches queued behind a spin, "
                                "after the timed steps")
    del dl
    t_cay = np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    t_fwd = np.mean([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    t_bwd = np.mean([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3
    f_fwd, f_bwd = moe_flops(cfg)
    by_fwd, by_bwd = moe_bytes(cfg, n_active)
    value = (f_fwd + f_bwd) / (wall / args.steps) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "experts": E, "top_k": k, "hidden": H,
                   "expert_intermediate": I, "weights": f"{cfg.w_fmt}_g{cfg.g}", "oft_block": b, "chunk": cfg.chunk,
                   "active_experts": n_active, "parallelism": "single_gpu"},
        "roofline": roofline_object((f_fwd + f_bwd) / (by_fwd + by_bwd) > RIDGE, f_fwd + f_bwd, by_fwd + by_bwd,
                                    t_fwd + t_bwd, kernel="moe fwd+bwd calls", traffic=None),
        "router_bwd": rb_roof,
        "phases_us": {"cayley_build": round(t_cay * 1e6, 2), "fwd": round(t_fwd * 1e6, 2),
                      "bwd": round(t_bwd * 1e6, 2)},
        "phase_rates": {"fwd_tflops": round(f_fwd / t_fwd / 1e12, 2), "bwd_tflops": round(f_bwd / t_bwd / 1e12, 2),
                        "fwd_alg_gbs": round(by_fwd / t_fwd / 1e9, 1), "bwd_alg_gbs": round(by_bwd / t_bwd / 1e9, 1),
                        "hbm_frac": round((by_fwd + by_bwd) / (t_fwd + t_bwd) / 1e9 / PEAK_HBM_GBS, 4)},
    }
    out["transient_bytes"] = int(transient)
    if not args.no_cold:
        cf, cb = cold_phases(
            lambda: oft.oft_moe_grouped_fwd(d, x, lg, W["wgu_codes"], W["wgu_scales"], W["wd_codes"], W["wd_scales"],
                                            Rops, rt, hs, y, wsf, nbf, stream=sp),
            lambda: oft.oft_moe_grouped_bwd(d, dy, rt, hs, W["wgu_codes"], W["wgu_scales"], W["wd_codes"],
                                            W["wd_scales"], Rf, Rops, dx, dq, dw, wsb, nbb, stream=sp))
        out["phases_cold_us"] = {"fwd": round(cf * 1e6, 2), "bwd": round(cb * 1e6, 2),
                                 "fwd_alg_gbs": round(by_fwd / cf / 1e9, 1), "bwd_alg_gbs": round(by_bwd / cb / 1e9, 1),
                                 "note": "fwd and bwd each right after writing 512 MiB (2x the MALL)"}
    if not args.no_dense_ref:
        del W
        out["dense_bf16_reference"] = moe_dense_reference(cfg, inp, args, dict(
            x=x, lg=lg, dy=dy, rt=rt, Rf=Rf, Rops=Rops, hs=hs, y=y, dx=dx, dq=dq, dw=dw), t_fwd + t_bwd)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = moe_cpu_baseline(cfg, inp)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    t_bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
    del wgu, wd, wsf, wsb
    torch.cuda.empty_cache()
    return {"fwd_us": round(t_fwd * 1e6, 2), "bwd_us": round(t_bwd * 1e6, 2),
            "weights_bytes": int(E * 3 * I * H * 2),
            "ratio": round(t_ours / (t_fwd + t_bwd), 4),
            "note": "fwd+bwd time of the INT4 path over that of the same kernels on bf16 weights"}


def moe_cpu_baseline(cfg, inp, n_experts=4):
    from oracle import moe as omoe

    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    idx, w = omoe.route(inp["logits"], cfg.k)
    rt = omoe.group(idx, cfg.E, cfg.chunk)
    rt.update(idx=idx, w=w)
    experts = [int(e) for e in rt["active"][:n_experts]]
    t0 = time.perf_counter()
    omoe.forward(inp, rt, experts=experts)
    omoe.backward(inp, rt, experts=experts)
    dt = time.perf_counter() - t0
    rows = int(sum(rt["counts"][e] for e in experts))
    H, I, b = cfg.H, cfg.I, cfg.b
    gemm = 2 * rows * H * 2 * I + 2 * rows * I * H
    fl = 2 * gemm + 6 * rows * 2 * I * b
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{cfg.name}: experts {experts} ({rows} routed rows), dequant + Cayley + fwd + bwd "
                      f"in fp64 numpy, {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; --gpus must be 1 "
                                   "(sharding over several GPUs is designed, not implemented)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import orthogonal_fine_tuning_amd as oft
    from oft_inputs import CONFIGS, make_dense

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = CONFIGS[args.config]
    if args.w_fmt is not None:
        if cfg.w_fmt not in ("int4", "fp4"):
            raise SystemExit(f"--w-fmt applies to 4-bit workloads; {cfg.name} has {cfg.w_fmt} weights")
        cfg = cfg.with_(w_fmt=args.w_fmt)
    if not hasattr(cfg, "segs"):
        print(json.dumps(run_moe(cfg, args)))
        return
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

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        oft.cayley_build(q, cfg.nblk, cfg.b, Rf, Rops, stream=sp)
        if ev is not None:
            ev[1].record(stream)
        oft.oft_linear_fwd(d, x, wc, ws, Rops, y, stream=sp)
        if ev is not None:
            ev[2].record(stream)
        oft.oft_linear_bwd(d, dy, y, wc, ws, Rf, Rops, dx, dq, work, nb, stream=sp)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_cay = np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    t_fwd = np.mean([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    t_bwd = np.mean([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3
    ms_per_step = wall / args.steps * 1e3

    # Roofline kernel time: one event pair on the same stream around a burst
    # of back-to-back forward launches (one kernel each), queued behind a
    # spin.  The per-phase
    # events above also count the idle time an event boundary adds on each
    # side of the launch it brackets (about 6 us here).
    burst = 10
    t_kernel = burst_seconds(stream, lambda: oft.oft_linear_fwd(d, x, wc, ws, Rops, y, stream=sp), burst)
    # the reference-policy forward (frozen base alone, oft_linear_fwd_base),
    # timed the same way
    t_base = burst_seconds(stream, lambda: oft.oft_linear_fwd_base(d, x, wc, ws, y, stream=sp), burst)
    # the forward on the active slot of a double-buffered adapter (one latch
    # launch, then the same kernels reading the slot through it)
    state = torch.zeros(4, dtype=torch.int32, device="cuda")
    latch = torch.zeros(4, dtype=torch.int32, device="cuda")
    oft.oft_slots_switch(state, 1, 1, stream=sp)
    # slot and plain bursts alternate three times and each side takes its
    # median: a single burst pair is at the mercy of where it falls in the
    # clock's response to sustained matrix-core load
    ts, tp = [], []
    for _ in range(3):
        ts.append(burst_seconds(stream, lambda: oft.oft_linear_fwd_slots(d, x, wc, ws, Rops, Rops, state, latch, y,
                                                                         stream=sp), burst))
        tp.append(burst_seconds(stream, lambda: oft.oft_linear_fwd(d, x, wc, ws, Rops, y, stream=sp), burst))
    t_slots, t_plain2 = float(np.median(ts)), float(np.median(tp))
    f_fwd, f_bwd = dense_flops(cfg)
    by_fwd, by_bwd = dense_bytes(cfg)
    value = (f_fwd + f_bwd) / (wall / args.steps) / 1e12

    fwd_src = FWD_KERNEL_SOURCES
    sha = kernel_source_sha(fwd_src)
    roof = roofline_object(f_fwd / by_fwd > RIDGE, f_fwd, by_fwd, t_kernel, kernel=fwd_kernel_name(cfg),
                           traffic=None if cfg.w_fmt != CONFIGS[args.config].w_fmt  # counters taken on the stock format
                           else load_traffic(f"{fwd_kernel_name(cfg)}:{cfg.name}", sha))
    roof["kernel_timing"] = f"HIP events around {burst} back-to-back launches queued behind a spin, after the timed steps"
    roof["source_sha"] = sha
    f_base = 2 * cfg.M * cfg.N * cfg.K
    by_base = by_fwd - cfg.nblk * 2 * cfg.b * cfg.b * 2  # no rotation operands
    base_roof = roofline_object(f_base / by_base > RIDGE, f_base, by_base, t_base, kernel=fwd_kernel_name(cfg),
                                traffic=None)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.M, "in_features": cfg.K,
                   "out_features": cfg.N, "segments": list(cfg.segs), "oft_block": cfg.b,
                   "weights": cfg.w_fmt + (f"_g{cfg.g}" if cfg.w_fmt != "fp8" else "_e4m3"),
                   "x_dtype": cfg.x_dtype, "parallelism": "single_gpu"},
        "roofline": roof,
        "reference_policy_fwd": base_roof,
        "slots_fwd": {"kernel_us": round(t_slots * 1e6, 2), "plain_fwd_us": round(t_plain2 * 1e6, 2),
                      "overhead_us": round((t_slots - t_plain2) * 1e6, 2),
                      "timing": "latch + forward per call, same burst timing as roofline; medians of three "
                                "slot bursts alternating with three plain-forward bursts"},
        "phases_us": {"cayley_build": round(t_cay * 1e6, 2), "fwd": round(t_fwd * 1e6, 2),
                      "bwd": round(t_bwd * 1e6, 2)},
        "phase_rates": {
            "fwd_tflops": round(f_fwd / t_fwd / 1e12, 2), "bwd_tflops": round(f_bwd / t_bwd / 1e12, 2),
            "fwd_alg_gbs": round(by_fwd / t_fwd / 1e9, 1), "bwd_alg_gbs": round(by_bwd / t_bwd / 1e9, 1),
            "step_mfma_frac": round(value / PEAK_BF16_TFLOPS, 4)},
    }
    if not args.no_cold:
        cf, cb = cold_phases(lambda: oft.oft_linear_fwd(d, x, wc, ws, Rops, y, stream=sp),
                             lambda: oft.oft_linear_bwd(d, dy, y, wc, ws, Rf, Rops, dx, dq, work, nb, stream=sp))
        out["phases_cold_us"] = {"fwd": round(cf * 1e6, 2), "bwd": round(cb * 1e6, 2),
                                 "fwd_alg_gbs": round(by_fwd / cf / 1e9, 1), "bwd_alg_gbs": round(by_bwd / cb / 1e9, 1),
                                 "note": "fwd and bwd each right after writing 512 MiB (2x the MALL)"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_rows)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
