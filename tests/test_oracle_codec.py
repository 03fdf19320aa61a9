"""Pins for the oracle's number formats: library casts and the format specs."""
import os

import numpy as np
import pytest
import torch

from oracle import codec, dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(codec.bf16_bits_to_f64(bits), ref)


def test_fp16_decode_exhaustive_vs_libraries():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref_np = bits.view(np.float16).astype(np.float64)
    ref_t = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    got = codec.fp16_bits_to_f64(bits)
    assert _same(got, ref_np)
    assert _same(got, ref_t)


def test_e4m3fn_decode_exhaustive_vs_torch():
    bits = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(codec.e4m3fn_bits_to_f64(bits), ref)


def test_e4m3fn_golden_spec_values():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e4m3fn_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    codes = np.array([int(r[0], 16) for r in rows], dtype=np.uint8)
    vals = np.array([float(r[1]) for r in rows])
    assert _same(codec.e4m3fn_bits_to_f64(codes), vals)


def test_bf16_rne_golden():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "bf16_rne.txt"))
            if ln.strip() and not ln.startswith("#")]
    src = np.array([int(r[0], 16) for r in rows], dtype=np.uint32).view(np.float32)
    want = np.array([int(r[1], 16) for r in rows], dtype=np.uint16)
    assert np.array_equal(codec.f32_to_bf16_bits(src), want)


def test_bf16_rne_vs_torch_random_and_ties():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # force a third of them onto exact ties and near-ties
    u[::3] = (u[::3] & 0xFFFF0000) | 0x8000
    u[1::3] = (u[1::3] & 0xFFFF0000) | rng.choice([0x7FFF, 0x8001], size=u[1::3].size)
    f = u.view(np.float32)
    finite = np.isfinite(f)
    f = f[finite]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codec.f32_to_bf16_bits(f), ref)


def test_int4_dequant_all_codes_vs_torch():
    """bf16_RNE(q * s) for all 16 codes x 1e5 random fp16 scales."""
    rng = np.random.default_rng(2)
    nscale = 100_000
    s_bits = rng.integers(0x0400, 0x7BFF, size=nscale).astype(np.uint16)  # normal fp16
    s_bits[: nscale // 2] = (np.float16(0.01) + rng.random(nscale // 2).astype(np.float16)
                             * np.float16(0.04)).view(np.uint16)
    # one row per scale, 16 columns = all nibbles 0..15 (two per byte)
    nib = np.arange(16, dtype=np.uint8)
    codes = np.broadcast_to(nib[0::2] | (nib[1::2] << 4), (nscale, 8)).copy()
    got = dense.dequant_int4(codes, s_bits[:, None], g=16)
    q = np.where(nib >= 8, nib.astype(np.int32) - 16, nib.astype(np.int32)).astype(np.float32)
    s32 = torch.from_numpy(s_bits.view(np.int16)).view(torch.float16).to(torch.float32)
    ref = (torch.from_numpy(q)[None, :] * s32[:, None]).to(torch.bfloat16).to(torch.float64)
    assert np.array_equal(got, ref.numpy())


def test_int4_nibble_order_and_sign():
    # byte 0x21: element 0 = low nibble 1, element 1 = high nibble 2
    # byte 0x8F: element 2 = 0xF -> -1, element 3 = 0x8 -> -8
    codes = np.array([[0x21, 0x8F]], dtype=np.uint8)
    assert dense.unpack_int4(codes).tolist() == [[1, 2, -1, -8]]
    one = np.float16(1.0).view(np.uint16)
    w = dense.dequant_int4(codes, np.array([[one]], dtype=np.uint16), g=4)
    assert w.tolist() == [[1.0, 2.0, -1.0, -8.0]]
    # group index follows the in-dim: scale 2 on the second group of 2
    two = np.float16(2.0).view(np.uint16)
    w = dense.dequant_int4(codes, np.array([[one, two]], dtype=np.uint16), g=2)
    assert w.tolist() == [[1.0, 2.0, -2.0, -16.0]]


# ---------------------------------------------------------------- FP4 (OCP MX)
def test_e2m1_golden_spec_values():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    codes = np.array([int(r[0], 16) for r in rows], dtype=np.uint8)
    vals = np.array([float(r[1]) for r in rows])
    assert len(codes) == 16 and sorted(codes.tolist()) == list(range(16))
    assert _same(codec.e2m1_bits_to_f64(codes), vals)


def test_e2m1_embeds_in_e4m3fn():
    """Every E2M1 value is an E4M3 value: moving the sign, re-biasing the
    exponent by 6 and widening the fraction gives the e4m3fn code of the
    same number (decoded by torch); the subnormals 0 and 0.5 map to 0 and
    2^-1."""
    c = np.arange(16, dtype=np.uint8)
    s, e, m = c >> 3, (c >> 1) & 3, c & 1
    e4 = np.where(e == 0, np.where(m == 1, 6, 0), e + 6)
    m4 = np.where(e == 0, 0, m << 2)
    code8 = ((s << 7) | (e4 << 3) | m4).astype(np.uint8)
    ref = torch.from_numpy(code8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(codec.e2m1_bits_to_f64(c), ref)
    assert np.all(np.diff(codec.e2m1_bits_to_f64(c[:8])) > 0)  # magnitudes increase with the code


def test_e8m0_values():
    c = np.array([0, 1, 126, 127, 128, 200, 254], dtype=np.uint8)
    assert np.array_equal(codec.e8m0_bits_to_f64(c), np.ldexp(1.0, c.astype(np.int64) - 127))
    assert np.isnan(codec.e8m0_bits_to_f64(np.array([255], dtype=np.uint8)))[0]


def test_fp4_dequant_nibble_order_groups_and_slot_byte():
    # byte 0x71: element 0 = low nibble 1 (0.5), element 1 = high nibble 7 (6)
    # byte 0xF8: element 2 = 0x8 (-0), element 3 = 0xF (-6)
    codes = np.array([[0x71, 0xF8]], dtype=np.uint8)
    w = dense.dequant_fp4(codes, np.array([[127]], dtype=np.uint16), g=4)
    assert _same(w, [[0.5, 6.0, -0.0, -6.0]])
    w = dense.dequant_fp4(codes, np.array([[127, 128]], dtype=np.uint16), g=2)  # 2^0, then 2^1
    assert _same(w, [[0.5, 6.0, -0.0, -12.0]])
    w = dense.dequant_fp4(codes, np.array([[0xAB7D]], dtype=np.uint16), g=4)  # high byte ignored: 2^-2
    assert _same(w, [[0.125, 1.5, -0.0, -1.5]])


def test_fp4_dequant_all_codes_all_exponents_vs_torch():
    """Every code under every finite exponent code: the exact product
    e2m1 * 2^(c - 127) (exactly representable in bf16, subnormals
    included), overflowing to infinity only where the magnitude reaches
    2^128; the same as torch's binary32 -> bf16 cast of the product."""
    nib = np.arange(16, dtype=np.uint8)
    codes = np.broadcast_to(nib[0::2] | (nib[1::2] << 4), (255, 8)).copy()
    slots = np.arange(255, dtype=np.uint16)[:, None]
    got = dense.dequant_fp4(codes, slots, g=16)
    exact = codec.e2m1_bits_to_f64(nib)[None, :] * np.ldexp(1.0, np.arange(255) - 127)[:, None]
    finite = np.abs(exact) < 2.0 ** 128
    assert _same(got[finite], exact[finite])
    # 2^128 and above: +-4 and +-6 at c = 253; +-2, +-3, +-4 and +-6 at c = 254
    assert (~finite).sum() == 12 and np.all(np.isinf(got[~finite]))
    assert np.array_equal(np.signbit(got[~finite]), np.signbit(exact[~finite]))
    with np.errstate(over="ignore"):
        e32 = exact.astype(np.float32)
    ref = torch.from_numpy(e32).to(torch.bfloat16).to(torch.float64).numpy()
    assert _same(got, ref)
