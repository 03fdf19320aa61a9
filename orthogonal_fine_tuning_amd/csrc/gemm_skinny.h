// Forward dequant GEMM for few tokens (decode batches, M <= 64):
//   C^T[n][m] = sum_k W[n][k] A[m][k]  + the same rotation epilogue as gemm_nt.h.
//
// At 64 tokens the layer is a weight stream: every weight byte is used by
// 64 tokens only, so the kernel is shaped for bytes in flight rather than
// matrix-core reuse.  A workgroup owns 32 channels (one 32-channel
// accumulator group = one b = 32 block or two b = 16 blocks) and 64 tokens;
// its 4 waves split K into quarters.  Weight bytes go HBM -> registers ->
// dequantised straight into matrix-core A operands (no LDS), two 64-wide K
// chunks of loads in flight per lane.  The contraction order inside a chunk
// is relabelled so that every lane reads 16 contiguous bytes of its weight
// row: in chunk c, MFMA j takes, for lane group g2, in-features
// k = c + 32 g2 + 8 j + p (p = item 0..7), and the token operand uses the
// same labels.  The 4 partial accumulators are summed through LDS in a fixed
// order, then wave 0 applies the FP8 scale, rounds to bf16, rotates
// (Y^T_blk = R_j Z^T_blk on the matrix cores; EPI_BASE: no rotation) and
// stores.
#pragma once

#include "gemm_nt.h"

namespace oft {

template <bool AF32, int WF, int B, bool OUTF32, int TN = 1, int EPI = EPI_ROT>
__global__ __launch_bounds__(256, 2) void gemm_nt_skinny_kernel(NtArgs p) {
  constexpr bool FP8 = WF == WF_FP8;
  static_assert(FP8 || wf_4bit(WF), "FP8 or 4-bit weights");
  static_assert(!wf_tiled(WF), "row-major weights only");
  static_assert(EPI == EPI_ROT || EPI == EPI_BASE, "epilogue");
  __shared__ float red[3][TN][2][16][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;
  const int nb0 = blockIdx.x * 32 * TN;
  const int m0 = blockIdx.y * 64;
  const int nrows = min(64, p.M - m0);
  const int kq = K / 4;
  const int kbeg = wave * kq;
  const int nchunk = kq / 64;
  const uint16_t* const rops = nt_rops(p);

  // weight rows of this lane: nb0 + 32 tn + l32 (always < N: N % (32 TN) == 0)
  const float* ws_f = static_cast<const float*>(p.ws);
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws);
  long xrow[2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int ml = tm * 32 + l32;
    xrow[tm] = ml < nrows ? (long)(m0 + ml) : -1;
  }

  struct Chunk {
    uint4 w[TN][FP8 ? 2 : 1];
    uint16_t s[TN];  // INT4: fp16 scale bits
    uint4 x[2][4][AF32 ? 2 : 1];
  };
  auto load = [&](Chunk& ch, int kc) {
    const int kk = kc + 32 * g2;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const size_t n = (size_t)(nb0 + 32 * tn + l32);
      if constexpr (FP8) {
        const uint8_t* src = p.wc + (size_t)n * K + kk;
        ch.w[tn][0] = *reinterpret_cast<const uint4*>(src);
        ch.w[tn][1] = *reinterpret_cast<const uint4*>(src + 16);
        ch.s[tn] = 0;
      } else {
        ch.w[tn][0] = *reinterpret_cast<const uint4*>(p.wc + (size_t)n * (K / 2) + kk / 2);
        ch.s[tn] = ws_h[n * (K / p.g) + kk / p.g];
      }
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (AF32) {
          const float* x = static_cast<const float*>(p.a) + xrow[tm] * p.lda + kk + 8 * j;
          ch.x[tm][j][0] = xrow[tm] >= 0 ? *reinterpret_cast<const uint4*>(x) : zero4();
          ch.x[tm][j][1] = xrow[tm] >= 0 ? *reinterpret_cast<const uint4*>(x + 4) : zero4();
        } else {
          const uint16_t* x = static_cast<const uint16_t*>(p.a) + xrow[tm] * p.lda + kk + 8 * j;
          ch.x[tm][j][0] = xrow[tm] >= 0 ? *reinterpret_cast<const uint4*>(x) : zero4();
        }
      }
  };

  f32x16 acc[TN][2];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tn][tm][r] = 0.0f;

  auto consume = [&](const Chunk& ch) {
    bf16x8 a[TN][4];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if constexpr (FP8) {
        const uint32_t wv[8] = {ch.w[tn][0].x, ch.w[tn][0].y, ch.w[tn][0].z, ch.w[tn][0].w,
                                ch.w[tn][1].x, ch.w[tn][1].y, ch.w[tn][1].z, ch.w[tn][1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 lo = dq_fp8x4(wv[2 * j]), hi = dq_fp8x4(wv[2 * j + 1]);
          a[tn][j] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
      } else {
        const auto sc = W4<WF>::scale(ch.s[tn]);
        a[tn][0] = as_bf16x8(W4<WF>::dq(ch.w[tn][0].x, sc));
        a[tn][1] = as_bf16x8(W4<WF>::dq(ch.w[tn][0].y, sc));
        a[tn][2] = as_bf16x8(W4<WF>::dq(ch.w[tn][0].z, sc));
        a[tn][3] = as_bf16x8(W4<WF>::dq(ch.w[tn][0].w, sc));
      }
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b;
        if constexpr (AF32) {
          const float4 u = __builtin_bit_cast(float4, ch.x[tm][j][0]);
          const float4 v = __builtin_bit_cast(float4, ch.x[tm][j][1]);
          b = as_bf16x8(make_uint4(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                                   pack_bf16x2(v.z, v.w)));
        } else {
          b = as_bf16x8(ch.x[tm][j][0]);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tn][tm] = mfma32(a[tn][j], b, acc[tn][tm]);
      }
  };

  // two chunks of loads in flight
  Chunk c0, c1;
  if (nchunk > 0) load(c0, kbeg);
  for (int c = 0; c < nchunk; c += 2) {
    if (c + 1 < nchunk) load(c1, kbeg + (c + 1) * 64);
    consume(c0);
    if (c + 1 < nchunk) {
      if (c + 2 < nchunk) load(c0, kbeg + (c + 2) * 64);
      consume(c1);
    }
  }

  // fixed-order reduction of the four K quarters
  if (wave > 0) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[wave - 1][tn][tm][r][lane] = acc[tn][tm][r];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[tn][tm][r] = ((acc[tn][tm][r] + red[0][tn][tm][r][lane]) + red[1][tn][tm][r][lane]) +
                         red[2][tn][tm][r][lane];

  // epilogue: FP8 scale, bf16, rotation on the matrix cores, store
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int nb = nb0 + 32 * tn;
    float sc[16];
    if constexpr (FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(ws_f + nb + 8 * q + 4 * g2);
        sc[4 * q] = v.x;
        sc[4 * q + 1] = v.y;
        sc[4 * q + 2] = v.z;
        sc[4 * q + 3] = v.w;
      }
    }
    bf16x8 ra[2];
    if constexpr (EPI == EPI_ROT) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint2 lo = make_uint2(0u, 0u), hi = make_uint2(0u, 0u);
        if constexpr (B == 32) {
          const uint16_t* Rj = rops + (size_t)(nb / 32) * 2048 + l32 * 32 + 16 * t + 4 * g2;
          lo = *reinterpret_cast<const uint2*>(Rj);
          hi = *reinterpret_cast<const uint2*>(Rj + 8);
        } else {
          if ((l32 >> 4) == t) {
            const uint16_t* Rj = rops + (size_t)(nb / 16 + t) * 512 + (l32 & 15) * 16 + 4 * g2;
            lo = *reinterpret_cast<const uint2*>(Rj);
            hi = *reinterpret_cast<const uint2*>(Rj + 8);
          }
        }
        ra[t] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      f32x16 z = acc[tn][tm];
      if constexpr (FP8) {
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] *= sc[r];
      }
      f32x16 o = z;
      if constexpr (EPI == EPI_ROT) {
        bf16x8 zb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          zb[t] = as_bf16x8(make_uint4(pack_bf16x2(z[8 * t], z[8 * t + 1]), pack_bf16x2(z[8 * t + 2], z[8 * t + 3]),
                                       pack_bf16x2(z[8 * t + 4], z[8 * t + 5]),
                                       pack_bf16x2(z[8 * t + 6], z[8 * t + 7])));
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = 0.0f;
        o = mfma32(ra[0], zb[0], o);
        o = mfma32(ra[1], zb[1], o);
      }
      const int ml = tm * 32 + l32;
      if (ml >= nrows) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t off = (size_t)(m0 + ml) * p.ldo + nb + 8 * q + 4 * g2;
        if constexpr (OUTF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off) =
              make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) =
              make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
        }
      }
    }
  }
}

}  // namespace oft
