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

// 8 INT4 nibbles (low nibble first) times one scale -> 8 bf16 (as uint4).
// Each product q*s is exact in fp32; the conversion rounds once (RNE).
__device__ __forceinline__ uint4 dq_int4x8(uint32_t w, float s) {
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int q = (int)(w << (28 - 4 * e)) >> 28;  // sign-extended nibble e
    f[e] = (float)q * s;
  }
  uint4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

// 4 e4m3fn bytes (byte 0 first) -> 4 bf16, exact (scale 1.0).
__device__ __forceinline__ uint2 dq_fp8x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// 4 nibbles (low first) of the low 16 bits of w times s -> 4 bf16 (uint2)
__device__ __forceinline__ uint2 dq_int4x4(uint32_t w, float s) {
  float f[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int q = (int)(w << (28 - 4 * e)) >> 28;
    f[e] = (float)q * s;
  }
  uint2 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

}  // namespace oft
