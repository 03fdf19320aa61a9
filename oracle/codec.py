"""Number formats, decoded from their bit-level definitions (fp64 results).

Test infrastructure only (see the package header).

* bf16: the upper half of an IEEE binary32 word; rounding fp32 -> bf16 is
  round-to-nearest-even on the discarded 16 bits.
* fp16: IEEE binary16 (1 sign, 5 exponent bits with bias 15, 10 fraction
  bits; exponent 0 is subnormal).
* e4m3fn: the OCP 8-bit float "E4M3" (1 sign, 4 exponent bits with bias 7,
  3 fraction bits; exponent 0 is subnormal; S.1111.111 is NaN; no infinity;
  largest finite 448).
* e2m1: the OCP Microscaling (MX) 4-bit float element "E2M1" (1 sign, 2
  exponent bits with bias 1, 1 fraction bit; exponent 0 is subnormal, value
  fraction / 2; no infinity or NaN; largest 6).
* e8m0: the OCP MX scale "E8M0" (8 exponent bits with bias 127, no sign, no
  fraction; 0xFF is NaN), the value 2^(code - 127).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen quietly
        return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); returns bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    r = np.where(nan, (u >> 16) | 0x40, r)  # keep NaNs quiet NaNs
    return r.astype(np.uint16)


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(u >> 15, -1.0, 1.0)
    e = (u >> 10) & 0x1F
    f = (u & 0x3FF).astype(np.float64)
    val = np.where(e == 0, f * 2.0 ** -24, (1024.0 + f) * np.exp2(e - 25.0))
    val = np.where(e == 31, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(u >> 7, -1.0, 1.0)
    e = (u >> 3) & 0xF
    f = (u & 0x7).astype(np.float64)
    val = np.where(e == 0, f * 2.0 ** -9, (8.0 + f) * np.exp2(e - 10.0))
    val = np.where((e == 15) & (f == 7), np.nan, val)
    return sign * val


def e2m1_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Low nibble of each value, decoded as OCP MX E2M1."""
    u = np.asarray(bits, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(u >> 3, -1.0, 1.0)
    e = (u >> 1) & 0x3
    f = (u & 0x1).astype(np.float64)
    val = np.where(e == 0, f * 0.5, (2.0 + f) * np.exp2(e - 2.0))
    return sign * val


def e8m0_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    return np.where(u == 0xFF, np.nan, np.exp2(u - 127.0))
