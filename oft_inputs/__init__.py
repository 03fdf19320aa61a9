"""Seeded synthetic inputs for the OFT dequant-GEMM path.

This module only draws random data and stores it in the encodings the
library consumes (bf16 / fp16 / e4m3fn bit patterns, packed INT4 nibbles).
It computes nothing of the method itself: no dequantisation, no Cayley map,
no GEMM.  Both the CPU oracle and the GPU path take their inputs from here,
so that they see identical bits.

Encodings (the library's documented layouts):
  * bf16 / fp16 tensors are numpy ``uint16`` arrays holding the bit pattern;
  * fp8 weights are ``uint8`` e4m3fn codes (OCP FP8: bias 7, max 448, no inf);
  * INT4 weights are ``uint8`` ``[N, K/2]``: byte ``k//2`` of row ``n`` holds
    element ``k`` in its low nibble when ``k`` is even and in its high nibble
    when ``k`` is odd; a nibble is a two's-complement integer in [-8, 7];
  * INT4 scales are fp16 ``[N, K/g]`` (one per row and group of ``g``
    consecutive in-features); FP8 scales are fp32 ``[N]``;
  * FP4 weights use the INT4 layout with OCP MX E2M1 codes in the nibbles;
    their scale slots are ``uint16`` ``[N, K/g]`` holding an E8M0 exponent
    code in the low byte;
  * adapter parameters are bf16 ``[nblk, b(b-1)/2]``: the strict upper
    triangle of each skew-symmetric block, row-major.

Shapes and distributions restate the five workloads of the OFT layer in the
Orbit pages (fused Q/K/V of a 4B model, gate/up of a 4B model at training and
decode token counts, a 30B-A3B MoE layer and one GPU's share of a ~1T MoE
layer).  Random numbers come from ``numpy.random.default_rng(seed)`` in a
fixed draw order, listed per generator below.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = [
    "DenseConfig",
    "MoEConfig",
    "CONFIGS",
    "make_dense",
    "make_moe",
    "make_moe_logits",
    "moe_token_rows",
    "to_bf16_bits",
    "to_fp16_bits",
]


# --------------------------------------------------------------------------
# encoders (library casts; these round inputs once, at generation time)
# --------------------------------------------------------------------------
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (round to nearest even, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_fp16_bits(a: np.ndarray) -> np.ndarray:
    """values -> IEEE fp16 bit patterns (round to nearest even, via numpy)."""
    return np.ascontiguousarray(a).astype(np.float16).view(np.uint16)


def _to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class DenseConfig:
    name: str
    M: int
    K: int
    segs: tuple
    b: int
    x_dtype: str  # "f32" | "bf16"
    w_fmt: str  # "int4" | "fp8" | "fp4"
    g: int = 0  # INT4 / FP4 group along the in-dim (0 for fp8)
    q_std: float = 0.02
    scale_lo: float = 0.01
    scale_hi: float = 0.05

    @property
    def N(self) -> int:
        return int(sum(self.segs))

    @property
    def nblk(self) -> int:
        return self.N // self.b

    @property
    def npair(self) -> int:
        return self.b * (self.b - 1) // 2

    def with_(self, **kw) -> "DenseConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    E: int
    k: int
    H: int
    I: int
    g: int
    chunk: int
    b: int
    q_std: float = 0.02
    bias_std: float = 0.0  # per-expert logit skew (0 = none)
    scale_lo: float = 0.01
    scale_hi: float = 0.05
    w_fmt: str = "int4"  # "int4" | "fp4"

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def nblk_e(self) -> int:
        """OFT blocks per expert (gate segment then up segment)."""
        return 2 * self.I // self.b

    @property
    def npair(self) -> int:
        return self.b * (self.b - 1) // 2

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    # tiny fused QKV: parity-only size the oracle finishes instantly
    "tiny_qkv": DenseConfig("tiny_qkv", M=64, K=256, segs=(128, 128, 128), b=16,
                            x_dtype="f32", w_fmt="int4", g=32, q_std=0.01),
    # fused QKV of a 4B-shaped model: 32x128 q heads, 8x128 k and v heads
    "qkv_4b": DenseConfig("qkv_4b", M=4096, K=2560, segs=(4096, 1024, 1024), b=32,
                          x_dtype="bf16", w_fmt="fp8", g=0, q_std=0.02),
    # fused gate/up of a 4B-shaped MLP, training token count and decode batch
    "gateup_4b_train": DenseConfig("gateup_4b_train", M=8192, K=2560, segs=(9728, 9728),
                                   b=32, x_dtype="bf16", w_fmt="int4", g=128),
    "gateup_4b_decode": DenseConfig("gateup_4b_decode", M=64, K=2560, segs=(9728, 9728),
                                    b=32, x_dtype="bf16", w_fmt="int4", g=128),
    # MoE layer shaped like a 30B-A3B model
    "moe_30b_a3b": MoEConfig("moe_30b_a3b", T=16384, E=128, k=8, H=2048, I=768, g=32,
                             chunk=8, b=32),
    # one GPU's share of a ~1T MoE layer, training and decode token counts
    "moe_1t_train": MoEConfig("moe_1t_train", T=4096, E=384, k=8, H=7168, I=2048, g=32,
                              chunk=16, b=32, bias_std=0.5),
    "moe_1t_decode": MoEConfig("moe_1t_decode", T=128, E=384, k=8, H=7168, I=2048, g=32,
                               chunk=16, b=32, bias_std=0.5),
}


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def _int4_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    """n bytes, each uniform over 0..255 (so each nibble is uniform over
    [-8, 7]): the little-endian bytes of ceil(n / 8) raw 64-bit outputs of
    the generator's bit stream, the first n of them."""
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n] if n % 8 else words.view(np.uint8)


def _scale_slots(rng: np.random.Generator, w_fmt: str, lo: float, hi: float, shape) -> np.ndarray:
    """INT4: fp16 scales uniform in [lo, hi].  FP4: E8M0 exponent codes
    uniform over those of the powers of two nearest lo and hi."""
    if w_fmt == "int4":
        return to_fp16_bits(rng.uniform(lo, hi, size=shape))
    c_lo, c_hi = 127 + int(np.round(np.log2(lo))), 127 + int(np.round(np.log2(hi)))
    return rng.integers(c_lo, c_hi + 1, size=shape).astype(np.uint16)


def make_dense(cfg: DenseConfig, seed: int = 0, with_dy: bool = True) -> dict:
    """Draw one dense OFT-linear problem.

    Draw order: x, weight (INT4 / FP4 codes | FP8 source values), weight scales,
    adapter parameters (segment by segment, block by block), dY.
    """
    rng = np.random.default_rng(seed)
    M, K, N, b = cfg.M, cfg.K, cfg.N, cfg.b
    out = {"cfg": cfg}
    xf = rng.standard_normal((M, K), dtype=np.float32)
    out["x"] = xf if cfg.x_dtype == "f32" else to_bf16_bits(xf)
    if cfg.w_fmt in ("int4", "fp4"):
        assert K % cfg.g == 0 and K % 2 == 0
        out["w_codes"] = _int4_bytes(rng, N * K // 2).reshape(N, K // 2)
        out["w_scales"] = _scale_slots(rng, cfg.w_fmt, cfg.scale_lo, cfg.scale_hi, (N, K // cfg.g))
    elif cfg.w_fmt == "fp8":
        w = rng.standard_normal((N, K), dtype=np.float32)
        s = (np.abs(w).max(axis=1) / np.float32(448.0)).astype(np.float32)
        out["w_codes"] = _to_e4m3_codes(w / s[:, None])
        out["w_scales"] = s
    else:
        raise ValueError(cfg.w_fmt)
    p = rng.normal(0.0, cfg.q_std, size=(cfg.nblk, cfg.npair)).astype(np.float32)
    out["p"] = to_bf16_bits(p)
    if with_dy:
        out["dy"] = to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
    return out


def make_moe(cfg: MoEConfig, seed: int = 0, with_dy: bool = True) -> dict:
    """Draw one MoE problem.

    Draw order: x, router logits, per-expert logit bias (only when
    ``bias_std > 0``; it is added to the logits in fp32 here, so consumers see
    biased logits only), gate/up codes, gate/up scales, down codes, down
    scales, adapter parameters (expert by expert, gate blocks then up blocks),
    dy.  Weights and scales are drawn expert by expert.
    """
    rng = np.random.default_rng(seed)
    T, E, H, I, g, b = cfg.T, cfg.E, cfg.H, cfg.I, cfg.g, cfg.b
    assert H % g == 0 and I % g == 0
    out = {"cfg": cfg}
    out["x"] = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if cfg.bias_std > 0:
        bias = rng.normal(0.0, cfg.bias_std, size=E).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
    out["logits"] = logits
    # expert by expert within each array: one draw per array is the same
    # stream as E consecutive per-expert draws (each a multiple of 8 bytes)
    wgu = _int4_bytes(rng, E * 2 * I * H // 2).reshape(E, 2 * I, H // 2)
    sgu = _scale_slots(rng, cfg.w_fmt, cfg.scale_lo, cfg.scale_hi, (E, 2 * I, H // g))
    wd = _int4_bytes(rng, E * H * I // 2).reshape(E, H, I // 2)
    sd = _scale_slots(rng, cfg.w_fmt, cfg.scale_lo, cfg.scale_hi, (E, H, I // g))
    out.update(wgu_codes=wgu, wgu_scales=sgu, wd_codes=wd, wd_scales=sd)
    p = rng.normal(0.0, cfg.q_std, size=(E, cfg.nblk_e, cfg.npair)).astype(np.float32)
    out["p"] = to_bf16_bits(p)
    if with_dy:
        out["dy"] = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    return out


def make_moe_logits(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """The router logits of ``make_moe(cfg, seed)`` without drawing the weights
    (same stream: x first, then logits, then the optional bias)."""
    rng = np.random.default_rng(seed)
    rng.standard_normal((cfg.T, cfg.H), dtype=np.float32)
    logits = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.bias_std > 0:
        bias = rng.normal(0.0, cfg.bias_std, size=cfg.E).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
    return logits


def moe_token_rows(inp: dict, cfg: MoEConfig) -> dict:
    """A problem of T = cfg.T tokens from a drawn one with at least as many:
    the same weights, adapter and expert layout, and its first T rows of x,
    logits and dy (each row is an independent draw of the same
    distribution, so this is a seeded problem of the smaller shape)."""
    src = inp["cfg"]
    assert (src.E, src.k, src.H, src.I, src.g, src.b, src.w_fmt) == (cfg.E, cfg.k, cfg.H, cfg.I, cfg.g, cfg.b,
                                                                     cfg.w_fmt) and cfg.T <= src.T
    out = dict(inp)
    out["cfg"] = cfg
    for key in ("x", "logits", "dy"):
        if key in inp:
            out[key] = inp[key][:cfg.T]
    return out
