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
