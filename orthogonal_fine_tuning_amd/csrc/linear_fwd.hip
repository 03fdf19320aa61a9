// Forward of the OFT linear layer: y = rot_R(x . dequant(W0)^T).
//
// Orbit pages: the base weight stays at deployment precision (chooseai.io
// release news, "Technical principles") and fused projections get one
// independent rotation per sub-projection, applied by custom split-projection
// kernels ("Five design features of the adapter-first architecture").
//
// One workgroup (4 waves) computes a 128 (channels n) x 256 (tokens m) tile
// of Z^T = W . x^T with bf16 matrix-core MFMA 32x32x16 and fp32 accumulators:
//   * x tile [256 x 64] is loaded to registers one K step ahead, converted to
//     bf16 (fp32 input) and stored to LDS;
//   * the W tile [128 x 64] is loaded packed (INT4: 16 B per thread, FP8:
//     32 B), dequantised in registers (INT4: bf16_RNE(q*s), FP8: exact
//     e4m3 -> bf16) and stored to LDS; the dequantised weight never touches
//     HBM;
//   * epilogue: the FP8 per-channel scale multiplies the accumulators, which
//     are rounded to bf16 and fed, still in registers, as the B operand of
//     two more MFMAs with R_j (bf16) as the A operand: Y^T_blk = R_j Z^T_blk.
//     A 32-channel accumulator group is exactly one b = 32 block (or two
//     b = 16 blocks, handled with a block-diagonal 32 x 32 operand), and
//     blocks never straddle projection segments, so every segment gets its
//     own rotation with no extra pass over HBM.
#include "oft_device.h"
#include "oft_launch.h"

namespace oft {
namespace {

constexpr int BM = 256;  // tokens per tile
constexpr int BN = 128;  // channels per tile
constexpr int BK = 64;   // contraction step
constexpr int LDK = BK + 8;

template <bool XF32, bool FP8, int B>
__global__ __launch_bounds__(256, 2) void linear_fwd_kernel(
    const void* __restrict__ xv, const uint8_t* __restrict__ wc, const void* __restrict__ wsv,
    const uint16_t* __restrict__ Rops, void* __restrict__ yv, int M, int K, int N, int g) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int wn = wave >> 1, wm = wave & 1;

  // ---------------- global -> register prefetch
  constexpr int XR = XF32 ? 16 : 8;
  uint4 xr[XR];
  uint4 wr[FP8 ? 2 : 1];
  float wsc = 0.0f;

  const int w_row = tid >> 1, w_half = tid & 1;
  const bool w_ok = (n0 + w_row) < N;

  auto load_tiles = [&](int k0) {
    if constexpr (XF32) {
      const float* x = static_cast<const float*>(xv);
      const int c = tid & 15;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int r = (tid >> 4) + 16 * i;
        const int m = m0 + r;
        xr[i] = m < M ? *reinterpret_cast<const uint4*>(x + (size_t)m * K + k0 + 4 * c) : zero4();
      }
    } else {
      const uint16_t* x = static_cast<const uint16_t*>(xv);
      const int c = tid & 7;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int m = m0 + r;
        xr[i] = m < M ? *reinterpret_cast<const uint4*>(x + (size_t)m * K + k0 + 8 * c) : zero4();
      }
    }
    const size_t n = (size_t)(n0 + w_row);
    if constexpr (FP8) {
      const uint8_t* src = wc + n * K + k0 + 32 * w_half;
      wr[0] = w_ok ? *reinterpret_cast<const uint4*>(src) : zero4();
      wr[1] = w_ok ? *reinterpret_cast<const uint4*>(src + 16) : zero4();
    } else {
      const uint8_t* src = wc + n * (K / 2) + k0 / 2 + 16 * w_half;
      wr[0] = w_ok ? *reinterpret_cast<const uint4*>(src) : zero4();
      const uint16_t* s = static_cast<const uint16_t*>(wsv);
      wsc = w_ok ? fp16_to_f32(s[n * (K / g) + (k0 + 32 * w_half) / g]) : 0.0f;
    }
  };

  auto store_tiles = [&]() {
    if constexpr (XF32) {
      const int c = tid & 15;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int r = (tid >> 4) + 16 * i;
        const float4 v = __builtin_bit_cast(float4, xr[i]);
        uint2 p;
        p.x = pack_bf16x2(v.x, v.y);
        p.y = pack_bf16x2(v.z, v.w);
        *reinterpret_cast<uint2*>(&Xs[r * LDK + 4 * c]) = p;
      }
    } else {
      const int c = tid & 7;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int r = (tid >> 3) + 32 * i;
        *reinterpret_cast<uint4*>(&Xs[r * LDK + 8 * c]) = xr[i];
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(&Ws[w_row * LDK + 32 * w_half]);
    if constexpr (FP8) {
      const uint32_t wv[8] = {wr[0].x, wr[0].y, wr[0].z, wr[0].w,
                              wr[1].x, wr[1].y, wr[1].z, wr[1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 lo = dq_fp8x4(wv[2 * e]), hi = dq_fp8x4(wv[2 * e + 1]);
        dst[e] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    } else {
      dst[0] = dq_int4x8(wr[0].x, wsc);
      dst[1] = dq_int4x8(wr[0].y, wsc);
      dst[2] = dq_int4x8(wr[0].z, wsc);
      dst[3] = dq_int4x8(wr[0].w, wsc);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  load_tiles(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (k0 + BK < K) load_tiles(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        a[tn] = *reinterpret_cast<const bf16x8*>(&Ws[(wn * 64 + tn * 32 + l32) * LDK + kk * 16 + 8 * g2]);
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        b[tm] = *reinterpret_cast<const bf16x8*>(&Xs[(wm * 128 + tm * 32 + l32) * LDK + kk * 16 + 8 * g2]);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) acc[tn][tm] = mfma32(a[tn], b[tm], acc[tn][tm]);
    }
  }

  // ---------------- epilogue: scale (FP8), rotate, store
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const int nb = n0 + wn * 64 + tn * 32;  // first channel of this 32-group
    if (nb >= N) continue;
    float sc[16];
    if constexpr (FP8) {
      const float* s = static_cast<const float*>(wsv);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(s + nb + 8 * q + 4 * g2);
        sc[4 * q] = v.x;
        sc[4 * q + 1] = v.y;
        sc[4 * q + 2] = v.z;
        sc[4 * q + 3] = v.w;
      }
    }
    // A operand: R rows j = l32; items follow the accumulator row order
    // i(t, p) = 16t + 8(p/4) + 4g2 + p%4.
    bf16x8 ra[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint2 lo = make_uint2(0u, 0u), hi = make_uint2(0u, 0u);
      if constexpr (B == 32) {
        const uint16_t* Rj = Rops + (size_t)(nb / 32) * 2 * 1024 + l32 * 32 + 16 * t + 4 * g2;
        lo = *reinterpret_cast<const uint2*>(Rj);
        hi = *reinterpret_cast<const uint2*>(Rj + 8);
      } else {
        if ((l32 >> 4) == t) {
          const uint16_t* Rj = Rops + (size_t)(nb / 16 + t) * 2 * 256 + (l32 & 15) * 16 + 4 * g2;
          lo = *reinterpret_cast<const uint2*>(Rj);
          hi = *reinterpret_cast<const uint2*>(Rj + 8);
        }
      }
      ra[t] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
      f32x16 z = acc[tn][tm];
      if constexpr (FP8) {
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] *= sc[r];
      }
      bf16x8 zb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        zb[t] = as_bf16x8(make_uint4(pack_bf16x2(z[8 * t], z[8 * t + 1]),
                                     pack_bf16x2(z[8 * t + 2], z[8 * t + 3]),
                                     pack_bf16x2(z[8 * t + 4], z[8 * t + 5]),
                                     pack_bf16x2(z[8 * t + 6], z[8 * t + 7])));
      f32x16 o;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = 0.0f;
      o = mfma32(ra[0], zb[0], o);
      o = mfma32(ra[1], zb[1], o);
      const int m = m0 + wm * 128 + tm * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t off = (size_t)m * N + nb + 8 * q + 4 * g2;
        if constexpr (XF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(yv) + off) =
              make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(yv) + off) =
              make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
        }
      }
    }
  }
}

template <bool XF32, bool FP8, int B>
hipError_t launch_fwd_t(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws,
                        const uint16_t* Rops, void* y, hipStream_t st) {
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  hipLaunchKernelGGL((linear_fwd_kernel<XF32, FP8, B>), grid, dim3(256), 0, st, x, wc, ws, Rops,
                     y, a.M, a.K, a.N, a.g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_fwd(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws,
                             const uint16_t* Rops, void* y, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
#define OFT_FWD_CASE(XF, F8, BB)                                   \
  if (a.xf32 == XF && a.fp8 == F8 && a.b == BB)                    \
    return launch_fwd_t<XF, F8, BB>(a, x, wc, ws, Rops, y, st);
  OFT_FWD_CASE(false, false, 32)
  OFT_FWD_CASE(false, false, 16)
  OFT_FWD_CASE(false, true, 32)
  OFT_FWD_CASE(false, true, 16)
  OFT_FWD_CASE(true, false, 32)
  OFT_FWD_CASE(true, false, 16)
  OFT_FWD_CASE(true, true, 32)
  OFT_FWD_CASE(true, true, 16)
#undef OFT_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace oft
