// Device-side helpers shared by the liboft kernels (gfx950 / CDNA4).
//
// Matrix-core operand layouts used throughout (v_mfma_f32_32x32x16_bf16,
// wave64, lane l, group g = l / 32):
//   A (32 x 16, rows i, contraction k): lane l holds row i = l % 32, items
//     p = 0..7 are k = 8g + p;
//   B (16 x 32, contraction k, cols j): lane l holds column j = l % 32,
//     items p are k = 8g + p;
//   C (32 x 32 fp32): lane l holds column j = l % 32, register r is row
//     i = (r / 4) * 8 + 4g + r % 4.
// Any consistent relabelling of k between A and B leaves the product
// unchanged; the rotation epilogues use that to feed an accumulator (C
// layout, rows in registers) straight back as a B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>
#include <utility>

#include "oft_formats.h"

namespace oft {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ __forceinline__ float fp16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// INT4 group scale in the forms the dequantisation uses (all exact in
// fp32: s has 11 significant bits, 1032 = 129 x 8 and 72 = 9 x 8): s and
// -1032 s for nibbles that sit in the low mantissa bits of an fp16, s / 16
// and -72 s for nibbles that sit four bits higher.
struct I4Scale {
  float s, m, s16, m16;
};
__device__ __forceinline__ I4Scale i4scale(uint16_t bits) {
  const float s = (float)__builtin_bit_cast(_Float16, bits);
  return I4Scale{s, -1032.0f * s, 0.0625f * s, -72.0f * s};
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 INT4 nibbles (low nibble first, two's complement) times one scale -> 8
// bf16 (as uint4), each bf16(q s) rounded once to nearest even.  A nibble n
// is moved into the mantissa of an fp16 whose exponent is 10 (value 1024 +
// mantissa) with its top bit flipped (n ^ 8 = q + 8), by one AND/XOR per two
// nibbles: nibbles 0 and 4 (bits 0-3 of each half) give 1024 + (q + 8),
// nibbles 1 and 5 (bits 4-7) give 1024 + 16 (q + 8) in place, and one shift
// by 8 bits brings nibbles 2, 6, 3 and 7 to the same positions.  A mixed
// fp16 x fp32 + fp32 FMA then yields (1024 + (q + 8)) s - 1032 s or
// (1024 + 16 (q + 8)) s / 16 - 72 s, both q s exactly (at most 15
// significant bits), rounded once to bf16 by the pack.
__device__ __forceinline__ uint4 dq_int4x8(uint32_t w, I4Scale sc) {
  const uint32_t v[2] = {w, w >> 8};
  float f[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const f16x2 lo = __builtin_bit_cast(f16x2, (v[j] & 0x000F000Fu) ^ 0x64086408u);  // nibbles 2j, 2j + 4
    const f16x2 hi = __builtin_bit_cast(f16x2, (v[j] & 0x00F000F0u) ^ 0x64806480u);  // nibbles 2j + 1, 2j + 5
    f[2 * j] = __builtin_fmaf((float)lo[0], sc.s, sc.m);
    f[2 * j + 4] = __builtin_fmaf((float)lo[1], sc.s, sc.m);
    f[2 * j + 1] = __builtin_fmaf((float)hi[0], sc.s16, sc.m16);
    f[2 * j + 5] = __builtin_fmaf((float)hi[1], sc.s16, sc.m16);
  }
  uint4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

// FP4 group scale: the E8M0 exponent code c in the low byte of the 16-bit
// slot stands for 2^(c - 127) (OCP Microscaling formats).  The conversion
// instruction takes the scale from the exponent field of an fp32 operand
// only, so c << 23 carries it exactly, c = 0 (2^-127) included.
__device__ __forceinline__ float fp4scale(uint16_t bits) {
  return __builtin_bit_cast(float, ((uint32_t)bits & 0xFFu) << 23);
}

// 8 E2M1 codes (low nibble first) times 2^(c - 127) -> 8 bf16
// (v_cvt_scalef32_pk_bf16_fp4, one byte = two codes per instruction; low
// nibble to the low half).  Exact: an E2M1 value has two significant bits,
// so the product only leaves the bf16 range by overflow (c >= 253), which
// gives infinity.
__device__ __forceinline__ uint4 dq_fp4x8(uint32_t w, float s) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  return r;
}

// The 4-bit formats behind one interface: W4<WF>::S the decoded group scale,
// scale(bits) its decode, dq(w, s) eight codes to bf16.  INT4 is the primary
// template so that code paths compiled but never taken for FP8 or bf16
// weights still name a type.
template <int WF>
struct W4 {
  using S = I4Scale;
  static __device__ __forceinline__ S scale(uint16_t bits) { return i4scale(bits); }
  static __device__ __forceinline__ uint4 dq(uint32_t w, S s) { return dq_int4x8(w, s); }
};
template <>
struct W4<WF_FP4> {
  using S = float;
  static __device__ __forceinline__ S scale(uint16_t bits) { return fp4scale(bits); }
  static __device__ __forceinline__ uint4 dq(uint32_t w, S s) { return dq_fp4x8(w, s); }
};

// 4 e4m3fn bytes (byte 0 first) -> 4 bf16, exact (scale 1.0).
__device__ __forceinline__ uint2 dq_fp8x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Grouped launches (grid gx x gy, gy >= ntiles work-list entries): the
// column tile cx and work-list tile ty of this workgroup, false past the
// gx * ntiles real tiles.  The logical order L = ty * gx + cx is dealt to
// the eight XCDs in contiguous runs: the hardware hands workgroup b to XCD
// b % 8, and XCD x takes logical tiles [x n8 + min(x, rem), ...) in order,
// so the column tiles of a row tile (its gathered rows) and an expert's
// consecutive row tiles (its weights) meet in one XCD's L2 (measured: MoE
// steps 4-9 % shorter than with workgroup b on logical tile b).
__device__ __forceinline__ bool grouped_tile(int ntiles, int& cx, int& ty) {
  const int gx = gridDim.x;
  const long total = (long)gx * ntiles;
  const long b = (long)blockIdx.y * gx + blockIdx.x;
  if (b >= total) return false;
  const int x = (int)(b & 7);
  const long slot = b >> 3, n8 = total >> 3;
  const int rem = (int)(total & 7);
  const long L = (long)x * n8 + (x < rem ? x : rem) + slot;
  ty = (int)(L / gx);
  cx = (int)(L % gx);
  return true;
}

// Steps 0 .. n-1 of a loop over an NST-deep LDS ring, unrolled by NST:
// f(s, integral_constant<int, s % NST>), so that each step's ring stage is a
// compile-time constant (its byte offset the LDS instructions' immediate).
template <int NST, class F, int... I>
__device__ __forceinline__ void ring_steps_impl(int n, F& f, std::integer_sequence<int, I...>) {
  for (int s = 0; s < n; s += NST) ((s + I < n ? (f(s + I, std::integral_constant<int, I>{}), 0) : 0), ...);
}
template <int NST, class F>
__device__ __forceinline__ void ring_steps(int n, F f) {
  ring_steps_impl<NST>(n, f, std::make_integer_sequence<int, NST>{});
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Cayley gradient of a group of G = 1024 / B^2 consecutive blocks (one for
// B = 32, four for B = 16): Gq = (R^T + I) S (I + R) / 2, dp_il = Gq_il -
// Gq_li (packed upper triangle, row-major).  Each of the 256
// threads owns four adjacent outputs of one block row, so every global load
// of the group is in flight at once; load_s(g, r, c) returns S[r][c .. c + 3]
// of block g.  lds holds 3 G B (B + 4) floats; nb <= G blocks are valid.
template <int B, class LoadS>
__device__ __forceinline__ void cayley_grad_group(float* lds, const float* __restrict__ Rg,
                                                  float* __restrict__ dqg, int nb, int tid, LoadS load_s) {
  constexpr int G = 1024 / (B * B), P = B + 4, BQ = B / 4, BS = B * P;
  constexpr int NP = B * (B - 1) / 2;
  const int g = tid / (B * BQ), r = (tid / BQ) % B, c = 4 * (tid % BQ);
  const bool ok = g < nb;
  float* S = lds + g * BS;               // S, later Gq
  float* Rm = lds + G * BS + g * BS;     // R
  float* T1 = lds + 2 * G * BS + g * BS;  // S (I + R)
  float4 rv = make_float4(0.f, 0.f, 0.f, 0.f), sv = rv;
  if (ok) {
    rv = *reinterpret_cast<const float4*>(Rg + (size_t)g * B * B + r * B + c);
    sv = load_s(g, r, c);
  }
  *reinterpret_cast<float4*>(Rm + r * P + c) = rv;
  *reinterpret_cast<float4*>(S + r * P + c) = sv;
  __syncthreads();
  float4 t = sv;  // T1 = S + S R
#pragma unroll
  for (int i = 0; i < B; i += 4) {
    const float4 sr = *reinterpret_cast<const float4*>(S + r * P + i);
    const float sk[4] = {sr.x, sr.y, sr.z, sr.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 rr = *reinterpret_cast<const float4*>(Rm + (i + j) * P + c);
      t.x += sk[j] * rr.x;
      t.y += sk[j] * rr.y;
      t.z += sk[j] * rr.z;
      t.w += sk[j] * rr.w;
    }
  }
  *reinterpret_cast<float4*>(T1 + r * P + c) = t;
  __syncthreads();
  float4 q = t;  // Gq = (T1 + R^T T1) / 2
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const float ri = Rm[i * P + r];
    const float4 tt = *reinterpret_cast<const float4*>(T1 + i * P + c);
    q.x += ri * tt.x;
    q.y += ri * tt.y;
    q.z += ri * tt.z;
    q.w += ri * tt.w;
  }
  // S is no longer read (its last reads precede the barrier above)
  const float gq[4] = {0.5f * q.x, 0.5f * q.y, 0.5f * q.z, 0.5f * q.w};
  *reinterpret_cast<float4*>(S + r * P + c) = make_float4(gq[0], gq[1], gq[2], gq[3]);
  __syncthreads();
  // dp_rl = Gq_rl - Gq_lr for this thread's entries l = c .. c + 3 above the
  // diagonal of row r: packed index r B - r (r + 1) / 2 + l - r - 1
  if (ok) {
    const int base = r * B - r * (r + 1) / 2 - r - 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int l = c + k;
      if (l > r) dqg[(size_t)g * NP + base + l] = gq[k] - S[l * P + r];
    }
  }
}

}  // namespace oft
