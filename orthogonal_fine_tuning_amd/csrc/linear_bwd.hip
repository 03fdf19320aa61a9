// Backward of the OFT linear layer.
//
//   dX = rot_R^T(dY) . dequant(W0)        (no gradient of the frozen base:
//                                           the Synced article on Orbit,
//                                           "Technical details", bypasses the
//                                           base-weight gradient GEMM)
//   dQ: S_j = dY_blk^T Y_blk, G_j = S_j R_j (= dY_blk^T Z_blk, Z = Y R),
//       dL/dQ_j = (R_j^T + I) G_j (R_j^T + I) / 2, packed dp_il = Gq_il - Gq_li.
//
// dX kernel: one workgroup computes a 128 (k) x 256 (tokens) tile of dX^T.
// Each contraction step covers 64 output channels n:
//   * prologue: dZ^T = R_j^T dY^T for the step's blocks on the matrix cores,
//     dY read straight from HBM in B-operand layout; FP8 multiplies by s_n;
//     rounded to bf16 into LDS;
//   * the W tile [64 n x 128 k] is loaded packed, dequantised in registers
//     and stored transposed (k-major, n contiguous) to LDS;
//   * main MFMAs dX^T += W^T dZ^T.
// dQ: stage 1 transposes 64 x 64 tiles of dY and Y through LDS and forms the
// b x b cross products S on the matrix cores, one fp32 partial per M slice;
// stage 2 reduces the slices in a fixed order and applies the Cayley
// gradient in fp32 with R_f32.
#include "oft_device.h"
#include "oft_launch.h"

namespace oft {
namespace {

constexpr int BKO = 128;  // output in-features per tile
constexpr int BNS = 64;   // channels per contraction step
constexpr int LDN = BNS + 8;

// WsT row k keeps channel n at column n ^ wsw(k): rows 8..15 of every 16
// swap their two 32-channel halves, so the transposed 8-byte stores of a
// half-wave (4 rows x 64 bytes) spread over all banks, while 16-byte operand
// reads stay contiguous.
__device__ __forceinline__ int wsw(int k) { return ((k >> 3) & 1) << 5; }

template <bool XF32, bool FP8, int B, int BM>
__global__ __launch_bounds__(256, 2) void linear_bwd_dx_kernel(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ wc, const void* __restrict__ wsv,
    const uint16_t* __restrict__ Rops, void* __restrict__ dxv, int M, int K, int N, int g) {
  __shared__ __attribute__((aligned(16))) uint16_t WsT[BKO * LDN];  // [k][n]
  __shared__ __attribute__((aligned(16))) uint16_t dZs[BM * LDN];   // [m][n]
  static_assert(BM == 128 || BM == 256, "tile");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int k0 = blockIdx.x * BKO, m0 = blockIdx.y * BM;
  const int wk = wave >> 1, wm = wave & 1;
  constexpr int TM = BM / 64;   // 32-token tiles per wave
  constexpr int PM = BM / 128;  // 32-token tiles each wave rotates in the prologue

  // W tile: thread owns rows n0 + 4*rg + q (q < 4), in-features k0 + 8*kg + e
  // (e < 8).  A wave covers 4 kg x 16 rg, so each transposed LDS write of a
  // wave fills 4 whole 128-byte rows (no bank conflicts); lanes 4j..4j+3
  // read 16 contiguous bytes of one row.
  const int kg = (tid & 3) + 4 * (tid >> 6), rg = (tid >> 2) & 15;
  const bool k_ok = (k0 + 8 * kg) < K;
  uint32_t wr32[4];  // INT4: 8 nibbles per row
  uint2 wr64[4];     // FP8: 8 bytes per row
  float wsc[4];

  // prologue operands: this wave rotates token tiles mt = PM*wave + i (i < PM)
  uint4 dyf[PM][2][2];  // [i][32-channel group][t]
  uint4 rtf[2][2];     // [32-channel group][t]
  float4 scf[2][4];    // FP8 channel scales of the step, C-layout order

  auto prefetch = [&](int n0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 4 * rg + q;
      const bool ok = k_ok && n < N;
      if constexpr (FP8) {
        wr64[q] = ok ? *reinterpret_cast<const uint2*>(wc + (size_t)n * K + k0 + 8 * kg)
                     : make_uint2(0u, 0u);
      } else {
        wr32[q] = ok ? *reinterpret_cast<const uint32_t*>(wc + (size_t)n * (K / 2) + (k0 + 8 * kg) / 2)
                     : 0u;
        const uint16_t* s = static_cast<const uint16_t*>(wsv);
        wsc[q] = ok ? fp16_to_f32(s[(size_t)n * (K / g) + (k0 + 8 * kg) / g]) : 0.0f;
      }
    }
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const int nb = n0 + 32 * grp;
      const bool gok = nb < N;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint4 v = zero4();
        if (gok) {
          if constexpr (B == 32) {
            v = *reinterpret_cast<const uint4*>(Rops + (size_t)(nb / 32) * 2048 + 1024 + l32 * 32 +
                                                16 * t + 8 * g2);
          } else {
            if ((l32 >> 4) == t)
              v = *reinterpret_cast<const uint4*>(Rops + (size_t)(nb / 16 + t) * 512 + 256 +
                                                  (l32 & 15) * 16 + 8 * g2);
          }
        }
        rtf[grp][t] = v;
        if constexpr (FP8) {
          if (t == 0) {
            const float* s = static_cast<const float*>(wsv);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              scf[grp][q] = gok ? *reinterpret_cast<const float4*>(s + nb + 8 * q + 4 * g2)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int i = 0; i < PM; ++i) {
          const int m = m0 + (PM * wave + i) * 32 + l32;
          dyf[i][grp][t] = (gok && m < M)
                               ? *reinterpret_cast<const uint4*>(dy + (size_t)m * N + nb + 16 * t + 8 * g2)
                               : zero4();
        }
      }
    }
  };

  auto stage = [&]() {
    // W tile -> LDS, transposed: WsT[k][n]
    uint16_t v[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 d;
      if constexpr (FP8) {
        const uint2 lo = dq_fp8x4(wr64[q].x), hi = dq_fp8x4(wr64[q].y);
        d = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        d = dq_int4x8(wr32[q], wsc[q]);
      }
      const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[q][e] = (uint16_t)(dw[e >> 1] >> (16 * (e & 1)));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 p;
      p.x = (uint32_t)v[0][e] | ((uint32_t)v[1][e] << 16);
      p.y = (uint32_t)v[2][e] | ((uint32_t)v[3][e] << 16);
      const int k = 8 * kg + e;
      *reinterpret_cast<uint2*>(&WsT[k * LDN + ((4 * rg) ^ wsw(k))]) = p;
    }
    // prologue: dZ^T = R^T dY^T per 32-channel group, into dZs[m][n]
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      float sc[16];
      if constexpr (FP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sc[4 * q] = scf[grp][q].x;
          sc[4 * q + 1] = scf[grp][q].y;
          sc[4 * q + 2] = scf[grp][q].z;
          sc[4 * q + 3] = scf[grp][q].w;
        }
      }
#pragma unroll
      for (int i = 0; i < PM; ++i) {
        f32x16 o;
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = 0.0f;
        o = mfma32(as_bf16x8(rtf[grp][0]), as_bf16x8(dyf[i][grp][0]), o);
        o = mfma32(as_bf16x8(rtf[grp][1]), as_bf16x8(dyf[i][grp][1]), o);
        if constexpr (FP8) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[r] *= sc[r];
        }
        const int ml = (PM * wave + i) * 32 + l32;
        // Lane (m, g2) holds channels 8q + 4g2 + 0..3 in registers 4q..4q+3.
        // Swapping one 4-channel run with lane m + 32(1 - g2) leaves lane g2
        // with channels 16h + 8g2 + 0..7 of the pair q = 2h, 2h + 1.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint2 p0 = make_uint2(pack_bf16x2(o[8 * h], o[8 * h + 1]),
                                      pack_bf16x2(o[8 * h + 2], o[8 * h + 3]));
          const uint2 p1 = make_uint2(pack_bf16x2(o[8 * h + 4], o[8 * h + 5]),
                                      pack_bf16x2(o[8 * h + 6], o[8 * h + 7]));
          const uint2 snd = g2 ? p0 : p1;
          uint2 rcv;
          rcv.x = (uint32_t)__shfl_xor((int)snd.x, 32);
          rcv.y = (uint32_t)__shfl_xor((int)snd.y, 32);
          const uint4 v = g2 ? make_uint4(rcv.x, rcv.y, p1.x, p1.y) : make_uint4(p0.x, p0.y, rcv.x, rcv.y);
          *reinterpret_cast<uint4*>(&dZs[ml * LDN + 32 * grp + 16 * h + 8 * g2]) = v;
        }
      }
    }
  };

  f32x16 acc[2][TM];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  prefetch(0);
  for (int n0 = 0; n0 < N; n0 += BNS) {
    __syncthreads();
    stage();
    __syncthreads();
    if (n0 + BNS < N) prefetch(n0 + BNS);
#pragma unroll
    for (int kk = 0; kk < BNS / 16; ++kk) {
      bf16x8 a[2], b[TM];
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
      {
        const int k = wk * 64 + tk * 32 + l32;
        a[tk] = *reinterpret_cast<const bf16x8*>(&WsT[k * LDN + ((kk * 16 + 8 * g2) ^ wsw(k))]);
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        b[tm] = *reinterpret_cast<const bf16x8*>(&dZs[(wm * (BM / 2) + tm * 32 + l32) * LDN + kk * 16 + 8 * g2]);
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[tk][tm] = mfma32(a[tk], b[tm], acc[tk][tm]);
    }
  }

#pragma unroll
  for (int tk = 0; tk < 2; ++tk) {
    const int kb = k0 + wk * 64 + tk * 32;
    if (kb >= K) continue;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int m = m0 + wm * (BM / 2) + tm * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t off = (size_t)m * K + kb + 8 * q + 4 * g2;
        const f32x16& o = acc[tk][tm];
        if constexpr (XF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(dxv) + off) =
              make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dxv) + off) =
              make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------- dq stage 1
constexpr int LDM = 64 + 8;

// dYT / YT row n keeps token m at column m ^ msw(n) (16-token groups XORed by
// bits 3..4 of n): the transposed 4-byte stores of a wave hit every bank
// twice at most, 16-byte operand reads stay contiguous.
__device__ __forceinline__ int msw(int n) { return ((n >> 3) & 3) << 4; }

template <bool YF32>
__global__ __launch_bounds__(256) void dq_partial_kernel(const uint16_t* __restrict__ dy,
                                                         const void* __restrict__ yv,
                                                         float* __restrict__ part, int M, int N,
                                                         int rows_per_split, int ng32) {
  __shared__ __attribute__((aligned(16))) uint16_t dYT[64 * LDM];  // [n][m]
  __shared__ __attribute__((aligned(16))) uint16_t YT[64 * LDM];   // [n][m]
  __shared__ float red[2][64][17];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int n0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int m_lo = split * rows_per_split;
  const int m_hi = min(M, m_lo + rows_per_split);
  const int grp = wave & 1, kh = wave >> 1;

  const int c = tid & 7, rp = tid >> 3;  // 8 channels, rows 2rp and 2rp+1
  const bool c_ok = n0 + 8 * c < N;

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  for (int ms = m_lo; ms < m_hi; ms += 64) {
    uint4 d[2], y[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = ms + 2 * rp + h;
      const bool ok = c_ok && m < m_hi;
      d[h] = ok ? *reinterpret_cast<const uint4*>(dy + (size_t)m * N + n0 + 8 * c) : zero4();
      if constexpr (YF32) {
        const float* yf = static_cast<const float*>(yv) + (size_t)m * N + n0 + 8 * c;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (ok) {
          a = *reinterpret_cast<const float4*>(yf);
          b = *reinterpret_cast<const float4*>(yf + 4);
        }
        y[h] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                          pack_bf16x2(b.z, b.w));
      } else {
        y[h] = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(yv) + (size_t)m * N +
                                                    n0 + 8 * c)
                  : zero4();
      }
    }
    __syncthreads();
    {
      const uint32_t d0[4] = {d[0].x, d[0].y, d[0].z, d[0].w};
      const uint32_t d1[4] = {d[1].x, d[1].y, d[1].z, d[1].w};
      const uint32_t y0[4] = {y[0].x, y[0].y, y[0].z, y[0].w};
      const uint32_t y1[4] = {y[1].x, y[1].y, y[1].z, y[1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const uint32_t pd = ((d0[e >> 1] >> sh) & 0xFFFFu) | (((d1[e >> 1] >> sh) & 0xFFFFu) << 16);
        const uint32_t py = ((y0[e >> 1] >> sh) & 0xFFFFu) | (((y1[e >> 1] >> sh) & 0xFFFFu) << 16);
        const int n = 8 * c + e;
        *reinterpret_cast<uint32_t*>(&dYT[n * LDM + ((2 * rp) ^ msw(n))]) = pd;
        *reinterpret_cast<uint32_t*>(&YT[n * LDM + ((2 * rp) ^ msw(n))]) = py;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const int kk = 2 * kh + kq;
      const int n = 32 * grp + l32;
      const int mo = (16 * kk + 8 * g2) ^ msw(n);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&dYT[n * LDM + mo]);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&YT[n * LDM + mo]);
      acc = mfma32(a, b, acc);
    }
  }

  // fixed-order reduction of the two k-halves, then one partial per slice
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[grp][lane][r] = acc[r];
  }
  __syncthreads();
  if (kh == 0) {
    const int g32 = n0 / 32 + grp;
    if (g32 < ng32) {
      float* dst = part + ((size_t)split * ng32 + g32) * 1024;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (r / 4) * 8 + 4 * g2 + (r % 4);
        dst[row * 32 + l32] = acc[r] + red[grp][lane][r];
      }
    }
  }
}

// ---------------------------------------------------------------- dq stage 2
// Per block: S = sum of the slice partials (fixed order); with
// R (R^T + I) = I + R the Cayley gradient is
//   Gq = (R^T + I) S (I + R) / 2,  dp_il = Gq_il - Gq_li.
template <int B>
__global__ __launch_bounds__(256) void dq_final_kernel(const float* __restrict__ part, int nsplit,
                                                       int ng32, const float* __restrict__ Rf,
                                                       float* __restrict__ dq) {
  __shared__ float S[B][B + 1], Rm[B][B + 1], T1[B][B + 1];
  const int j = blockIdx.x;
  const int tid = threadIdx.x;
  const int g32 = (j * B) / 32, off = (j * B) % 32;
  for (int e = tid; e < B * B; e += 256) {
    const int r = e / B, c = e % B;
    float s = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp)
      s += part[((size_t)sp * ng32 + g32) * 1024 + (off + r) * 32 + off + c];
    S[r][c] = s;
    Rm[r][c] = Rf[(size_t)j * B * B + e];
  }
  __syncthreads();
  for (int e = tid; e < B * B; e += 256) {  // T1 = S (I + R)
    const int r = e / B, c = e % B;
    float s = S[r][c];
#pragma unroll 8
    for (int i = 0; i < B; ++i) s += S[r][i] * Rm[i][c];
    T1[r][c] = s;
  }
  __syncthreads();
  for (int e = tid; e < B * B; e += 256) {  // S = (R^T + I) T1 / 2
    const int r = e / B, c = e % B;
    float s = T1[r][c];
#pragma unroll 8
    for (int i = 0; i < B; ++i) s += Rm[i][r] * T1[i][c];
    S[r][c] = 0.5f * s;
  }
  __syncthreads();
  constexpr int NP = B * (B - 1) / 2;
  for (int pidx = tid; pidx < NP; pidx += 256) {
    // invert the row-major upper-triangle index
    int i = 0, rem = pidx;
    while (rem >= B - 1 - i) {
      rem -= B - 1 - i;
      ++i;
    }
    const int l = i + 1 + rem;
    dq[(size_t)j * NP + pidx] = S[i][l] - S[l][i];
  }
}

template <bool XF32, bool FP8, int B>
hipError_t launch_dx_t(const DenseArgs& a, const uint16_t* dy, const uint8_t* wc, const void* ws,
                       const uint16_t* Rops, void* dx, hipStream_t st) {
#ifndef OFT_DX_BM
#define OFT_DX_BM 128
#endif
  constexpr int BM = OFT_DX_BM;
  dim3 grid((a.K + BKO - 1) / BKO, (a.M + BM - 1) / BM);
  hipLaunchKernelGGL((linear_bwd_dx_kernel<XF32, FP8, B, BM>), grid, dim3(256), 0, st, dy, wc, ws,
                     Rops, dx, a.M, a.K, a.N, a.g);
  return hipGetLastError();
}

}  // namespace

DqPlan plan_dq(int M, int N) {
  DqPlan p;
  p.ng32 = N / 32;
  const int ng64 = (N + 63) / 64;
  const int msteps = (M + 63) / 64;
  int want = ng64 > 0 ? (1024 + ng64 - 1) / ng64 : 1;
  if (want < 1) want = 1;
  if (want > 16) want = 16;
  if (want > msteps) want = msteps;
  if (msteps == 0) {
    p.nsplit = 0;
    p.rows_per_split = 64;
  } else {
    const int steps_per = (msteps + want - 1) / want;
    p.rows_per_split = steps_per * 64;
    p.nsplit = (msteps + steps_per - 1) / steps_per;
  }
  p.part_bytes = (size_t)(p.nsplit > 0 ? p.nsplit : 1) * p.ng32 * 1024 * sizeof(float);
  return p;
}

hipError_t launch_linear_bwd_dx(const DenseArgs& a, const uint16_t* dy, const uint8_t* wc,
                                const void* ws, const uint16_t* Rops, void* dx, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
#define OFT_DX_CASE(XF, F8, BB) \
  if (a.xf32 == XF && a.fp8 == F8 && a.b == BB) return launch_dx_t<XF, F8, BB>(a, dy, wc, ws, Rops, dx, st);
  OFT_DX_CASE(false, false, 32)
  OFT_DX_CASE(false, false, 16)
  OFT_DX_CASE(false, true, 32)
  OFT_DX_CASE(false, true, 16)
  OFT_DX_CASE(true, false, 32)
  OFT_DX_CASE(true, false, 16)
  OFT_DX_CASE(true, true, 32)
  OFT_DX_CASE(true, true, 16)
#undef OFT_DX_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_linear_dq(const DenseArgs& a, const DqPlan& p, const uint16_t* dy, const void* y,
                            const float* Rf, float* dq, float* part, hipStream_t st) {
  if (p.nsplit > 0) {
    dim3 grid((a.N + 63) / 64, p.nsplit);
    if (a.xf32)
      hipLaunchKernelGGL(dq_partial_kernel<true>, grid, dim3(256), 0, st, dy, y, part, a.M, a.N,
                         p.rows_per_split, p.ng32);
    else
      hipLaunchKernelGGL(dq_partial_kernel<false>, grid, dim3(256), 0, st, dy, y, part, a.M, a.N,
                         p.rows_per_split, p.ng32);
  }
  const int nblk = a.N / a.b;
  if (a.b == 32)
    hipLaunchKernelGGL(dq_final_kernel<32>, dim3(nblk), dim3(256), 0, st, part, p.nsplit, p.ng32, Rf, dq);
  else
    hipLaunchKernelGGL(dq_final_kernel<16>, dim3(nblk), dim3(256), 0, st, part, p.nsplit, p.ng32, Rf, dq);
  return hipGetLastError();
}

}  // namespace oft
