"""Dense OFT linear layer over a frozen low-precision base, in fp64.

Test infrastructure only (see the package header).

Follows [P2] "Technical principles" (frozen INT4/FP8 base, BF16 OFT adapter),
[P2] "Five design features" / "OFT over LoRA" (an independent orthogonal
rotation for every sub-projection of a fused tensor) and [P1] "Technical
details" (the backward never forms a gradient for the frozen base).

Conventions (this library's readings; the pages print no formula):
  * INT4: element k of row n sits in byte k//2, low nibble for even k;
    two's complement, [-8, 7]; scale s[n, k//g] (fp16).  The dequantised
    weight is bf16_RNE(q * s): the product is exact in binary32, so this is a
    single rounding.
  * FP8: e4m3fn codes decode exactly; the per-row fp32 scale multiplies the
    row.  The oracle uses the exact product code * scale.
  * FP4 (the pages name an FP4 base but not its encoding; read as OCP MX):
    E2M1 codes in the INT4 nibble layout, and per group of g an E8M0
    exponent code in the low byte of a 16-bit slot (high byte ignored).  The
    dequantised weight is bf16_RNE(e2m1 * 2^(c - 127)): exact unless it
    overflows.
  * Adapter block j covers output channels [j*b, (j+1)*b) (segments are
    multiples of b and follow one another, so no block straddles two
    segments).  Q_j[i, l] = p, Q_j[l, i] = -p for the packed entry p of the
    pair (i, l), i < l, in row-major upper-triangle order.
  * y_blk = z_blk R_j^T (per token: y = R z).
"""
from __future__ import annotations

import numpy as np

from .codec import (bf16_bits_to_f64, e2m1_bits_to_f64, e4m3fn_bits_to_f64, e8m0_bits_to_f64, f32_to_bf16_bits,
                    fp16_bits_to_f64)


# ---------------------------------------------------------------- dequant
def unpack_int4(codes: np.ndarray) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] signed integers in [-8, 7]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    q = np.empty((rows, 2 * half), dtype=np.int16)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    return np.where(q >= 8, q - 16, q).astype(np.int8)


def dequant_int4(codes: np.ndarray, scale_bits: np.ndarray, g: int) -> np.ndarray:
    """W[n, k] = bf16_RNE(q[n, k] * s[n, k // g]) as fp64."""
    q = unpack_int4(codes).astype(np.float64)
    s = fp16_bits_to_f64(scale_bits)
    prod = q * np.repeat(s, g, axis=1)  # exact: <= 14 significant bits
    return bf16_bits_to_f64(f32_to_bf16_bits(prod.astype(np.float32)))


def unpack_fp4(codes: np.ndarray) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] E2M1 codes 0..15 (low nibble = even k)."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    c = np.empty((rows, 2 * half), dtype=np.uint8)
    c[:, 0::2] = codes & 0x0F
    c[:, 1::2] = codes >> 4
    return c


def dequant_fp4(codes: np.ndarray, scale_slots: np.ndarray, g: int) -> np.ndarray:
    """W[n, k] = bf16_RNE(e2m1(c[n, k]) * 2^(e[n, k // g] - 127)) as fp64,
    e the low byte of the 16-bit scale slot."""
    v = e2m1_bits_to_f64(unpack_fp4(codes))
    s = e8m0_bits_to_f64((np.asarray(scale_slots, dtype=np.uint16) & 0xFF).astype(np.uint8))
    prod = v * np.repeat(s, g, axis=1)  # exact in fp64: 2 significant bits
    with np.errstate(over="ignore"):  # 6 * 2^127 overflows binary32, as it overflows bf16
        return bf16_bits_to_f64(f32_to_bf16_bits(prod.astype(np.float32)))


def dequant_fmt(w_fmt: str, codes: np.ndarray, scales: np.ndarray, g: int) -> np.ndarray:
    """The dequantised base weight of one matrix in any of the formats."""
    if w_fmt == "int4":
        return dequant_int4(codes, scales, g)
    if w_fmt == "fp4":
        return dequant_fp4(codes, scales, g)
    if w_fmt == "fp8":
        return dequant_fp8(codes, scales)
    raise ValueError(w_fmt)


def dequant_fp8_codes(codes: np.ndarray) -> np.ndarray:
    """Exact e4m3fn values of the codes (the per-row scale is NOT applied)."""
    return e4m3fn_bits_to_f64(codes)


def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Full FP8 base weight: e4m3fn(code) * s[n], exact in fp64."""
    return dequant_fp8_codes(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def dequant(inp: dict) -> np.ndarray:
    cfg = inp["cfg"]
    return dequant_fmt(cfg.w_fmt, inp["w_codes"], inp["w_scales"], cfg.g)


# ---------------------------------------------------------------- Cayley
def skew(p: np.ndarray, b: int) -> np.ndarray:
    """Packed upper triangles (fp64 values) [nblk, b(b-1)/2] -> Q [nblk, b, b]."""
    p = np.asarray(p, dtype=np.float64).reshape(-1, b * (b - 1) // 2)
    Q = np.zeros((p.shape[0], b, b))
    iu, ju = np.triu_indices(b, 1)  # (0,1), (0,2), ..., (1,2), ...
    Q[:, iu, ju] = p
    Q[:, ju, iu] = -p
    return Q


def cayley_params(p: np.ndarray, b: int) -> np.ndarray:
    """R_j = (I + Q_j)(I - Q_j)^-1 for every block, fp64 [nblk, b, b]."""
    Q = skew(p, b)
    eye = np.broadcast_to(np.eye(b), Q.shape)
    return (eye + Q) @ np.linalg.solve(eye - Q, eye)


def cayley(p_bits: np.ndarray, b: int) -> np.ndarray:
    """Cayley map of bf16-encoded packed parameters."""
    return cayley_params(bf16_bits_to_f64(p_bits), b)


def pack_skew_grad(dLdQ: np.ndarray) -> np.ndarray:
    """Gradient w.r.t. the packed parameters: dp_il = dL/dQ_il - dL/dQ_li."""
    b = dLdQ.shape[-1]
    iu, ju = np.triu_indices(b, 1)
    return dLdQ[..., iu, ju] - dLdQ[..., ju, iu]


def cayley_grad(R: np.ndarray, G: np.ndarray) -> np.ndarray:
    """dL/dp from G = dL/dR.

    With A = I - Q, R = 2 A^-1 - I, so dR = 2 A^-1 dQ A^-1 and
    dL/dQ = 2 A^-T G A^-T; A^-1 = (R + I) / 2 gives
    dL/dQ = (R^T + I) G (R^T + I) / 2.
    """
    eye = np.eye(R.shape[-1])
    Rt = np.swapaxes(R, -1, -2) + eye
    return pack_skew_grad(0.5 * (Rt @ G @ Rt))


# ---------------------------------------------------------------- rotation
def rotate(Z: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Y_blk = Z_blk R_j^T for blocks of b consecutive columns."""
    M, N = Z.shape
    nblk, b, _ = R.shape
    Zb = Z.reshape(M, nblk, b)
    return np.einsum("mji,jri->mjr", Zb, R).reshape(M, N)


def rotate_adjoint(dY: np.ndarray, R: np.ndarray) -> np.ndarray:
    """dZ_blk = dY_blk R_j (adjoint of ``rotate``)."""
    M, N = dY.shape
    nblk, b, _ = R.shape
    return np.einsum("mjr,jri->mji", dY.reshape(M, nblk, b), R).reshape(M, N)


def rotation_grad(dY: np.ndarray, Z: np.ndarray, b: int) -> np.ndarray:
    """G_j = dY_blk^T Z_blk = dL/dR_j, [nblk, b, b]."""
    M, N = Z.shape
    return np.einsum("mjr,mji->jri", dY.reshape(M, N // b, b), Z.reshape(M, N // b, b))


# ---------------------------------------------------------------- layer
def x_f64(inp: dict) -> np.ndarray:
    cfg = inp["cfg"]
    if cfg.x_dtype == "f32":
        return np.asarray(inp["x"], dtype=np.float64)
    return bf16_bits_to_f64(inp["x"])


def forward(x: np.ndarray, W: np.ndarray, R: np.ndarray) -> np.ndarray:
    """y = rot_R(x W^T)."""
    return rotate(x @ W.T, R)


def base_forward(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """The frozen base alone, y = x W^T: the KL reference of [P2] "Five
    design features" (the reference policy is the base without the adapter,
    so no copy of the actor is kept)."""
    return x @ W.T


def backward(x: np.ndarray, W: np.ndarray, R: np.ndarray, dY: np.ndarray):
    """Gradients of <dY, y> w.r.t. x and the packed adapter parameters.

    dZ = rot^T(dY); dX = dZ W (no dW0: the base is frozen);
    G_j = dY_blk^T Z_blk; dp = cayley_grad(R, G).
    """
    b = R.shape[-1]
    Z = x @ W.T
    dZ = rotate_adjoint(dY, R)
    dX = dZ @ W
    dp = cayley_grad(R, rotation_grad(dY, Z, b))
    return dX, dp


def run(inp: dict) -> dict:
    """Whole dense problem from generator output: y, dX, dp, R (all fp64)."""
    cfg = inp["cfg"]
    W = dequant(inp)
    R = cayley(inp["p"], cfg.b)
    x = x_f64(inp)
    y = forward(x, W, R)
    out = {"R": R, "y": y}
    if "dy" in inp:
        dX, dp = backward(x, W, R, bf16_bits_to_f64(inp["dy"]))
        out.update(dx=dX, dp=dp)
    return out
