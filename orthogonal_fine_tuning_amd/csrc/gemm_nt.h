// Generic forward-type dequant GEMM:  C^T[n][m] = sum_k W[n][k] A[m][k]
// (W: packed 4-bit / FP8 rows, A: token rows), bf16 MFMA 32x32x16 with fp32
// accumulation, dequantisation in registers on the way into LDS.
//
// Row mapping:
//   dense   : tile y covers tokens [y*BM, y*BM + BM) of M;
//   grouped : tile y is entry y of a device work list (expert e, row0); its
//             rows are positions offsets[e] + row0 + r of the expert-sorted
//             order; the A row of a position is perm[pos] / kslots (gather of
//             the routed token) or the position itself (kslots == 0); the
//             weight, scale and rotation pointers advance by expert.
// Epilogues:
//   EPI_ROT        : (FP8 scale), round to bf16, Y^T_blk = R_j Z^T_blk on the
//                    matrix cores (accumulator registers reused directly as
//                    the B operand), store rows;
//   EPI_PLAIN      : (FP8 scale), store rows;
//   EPI_ROT_SWIGLU : channel tile = 64 gate channels [c, c+64) and the
//                    matching 64 up channels [I+c, I+c+64); both are rotated
//                    and stored, then act = silu(gate) * up (from the bf16
//                    values just stored) is written as well;
//   EPI_BASE       : FP8 scale, store rows (the frozen base alone, R = I);
//   EPI_BASE_SWIGLU: EPI_ROT_SWIGLU without the rotation (the frozen base
//                    alone); the h store is skipped when out is null.
#pragma once

#include "oft_device.h"

namespace oft {

enum : int { EPI_ROT = 0, EPI_PLAIN = 1, EPI_ROT_SWIGLU = 2, EPI_BASE = 3, EPI_BASE_SWIGLU = 4 };
// epilogues that apply the block rotation
constexpr bool epi_rotates(int epi) { return epi == EPI_ROT || epi == EPI_ROT_SWIGLU; }
// epilogues of the gate/up projection: gate and up channel halves, SwiGLU
constexpr bool epi_swiglu(int epi) { return epi == EPI_ROT_SWIGLU || epi == EPI_BASE_SWIGLU; }

struct NtArgs {
  const void* a;
  long lda;
  const uint8_t* wc;
  const void* ws;
  long wc_e, ws_e;  // per-expert strides: code bytes, scale elements
  const uint16_t* rops;
  long rops_e;      // per-expert stride of the rotation operands (elements)
  // double-buffered adapter: when rops_sel is set, *rops_sel (the slot
  // latched for this call) picks rops (0) or rops + rops_alt (1): the second
  // pack is addressed from the first, so every operand pointer stays derived
  // from the kernel argument
  long rops_alt;  // elements from rops to the second pack
  const int* rops_sel;
  void* out;
  long ldo;
  uint16_t* act;    // EPI_ROT_SWIGLU only
  long ldact;
  int M, K, N, g;
  int half_n;       // EPI_ROT_SWIGLU: I
  const int* tiles;   // grouped: [2 * max_tiles] (expert, row0)
  const int* ntiles;  // grouped: number of valid work-list entries
  const int* offsets;
  const int* perm;
  int kslots;
};

// the rotation operands of this launch (the latched slot of a
// double-buffered adapter, else rops)
__device__ __forceinline__ const uint16_t* nt_rops(const NtArgs& p) {
  const long off = (p.rops_sel != nullptr && *p.rops_sel == 1) ? p.rops_alt : 0;
  return p.rops + off;
}

namespace nt {
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;
}  // namespace nt

// Pipeline (NBUF = 2): two LDS buffers, registers one step ahead, one
// barrier per K step: while the matrix cores run step s from one buffer, the
// same waves dequantise step s + 1 (already in registers) into the other
// buffer and issue the global loads of step s + 2.  NBUF = 1: one buffer, two
// barriers per step; the smaller LDS footprint lets two workgroups share a
// CU and overlap each other's dequantisation with their matrix-core work.
template <int BM, bool AF32, int WF, int B, int EPI, bool GROUPED, bool OUTF32, int NBUF = 2>
__global__ __launch_bounds__(256, (BM == 256 && NBUF == 2) ? 1 : 2) void gemm_nt_kernel(NtArgs p) {
  using namespace nt;
  constexpr bool FP8 = WF == WF_FP8;
  static_assert(FP8 || wf_4bit(WF), "FP8 or 4-bit weights");
  static_assert(!wf_tiled(WF), "row-major weights only");
  static_assert(BM == 128 || BM == 256, "tile");
  static_assert(NBUF == 1 || NBUF == 2, "buffers");
  constexpr int TM = BM / 64;  // 32-token tiles per wave
  constexpr int STAGE = (BM + BN) * LDK;
  __shared__ __attribute__((aligned(16))) uint16_t smem[NBUF * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int wn = wave >> 1, wm = wave & 1;
  const int K = p.K;

  // ------------------------------------------------------------ tile setup
  int e = 0, pos0, nrows;
  if constexpr (GROUPED) {
    const int t = blockIdx.y;
    if (t >= *p.ntiles) return;
    e = p.tiles[2 * t];
    const int r0 = p.tiles[2 * t + 1];
    pos0 = p.offsets[e] + r0;
    nrows = min(BM, p.offsets[e + 1] - pos0);
  } else {
    pos0 = blockIdx.y * BM;
    nrows = min(BM, p.M - pos0);
  }
  const uint8_t* wc = p.wc + (size_t)e * p.wc_e;
  const uint16_t* rops = nt_rops(p) + (size_t)e * p.rops_e;
  const float* ws_f = static_cast<const float*>(p.ws);
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws) + (size_t)e * p.ws_e;

  auto a_row = [&](int r) -> long {
    if constexpr (GROUPED) {
      if (p.kslots > 0) return (long)(p.perm[pos0 + r] / p.kslots);
    }
    return (long)(pos0 + r);
  };
  // channel of local weight row w (0..BN-1)
  auto w_chan = [&](int w) -> int {
    if constexpr (EPI == EPI_ROT_SWIGLU) {
      const int c = blockIdx.x * (BN / 2);
      return w < BN / 2 ? c + w : p.half_n + c + (w - BN / 2);
    } else {
      return blockIdx.x * BN + w;
    }
  };

  // ------------------------------------------------------------ prefetch state
  constexpr int XR = AF32 ? 2 * BM / 32 : BM / 32;  // 16-byte loads per thread
  uint4 xr[XR];
  long xrow[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int r = AF32 ? (tid >> 4) + 16 * i : (tid >> 3) + 32 * i;
    xrow[i] = r < nrows ? a_row(r) : -1;
  }
  uint4 wr[FP8 ? 2 : 1];
  uint16_t wsb = 0;  // INT4: fp16 scale bits of the prefetched weight row
  const int w_row = tid >> 1, w_half = tid & 1;
  const int wchan = w_chan(w_row);
  const bool w_ok = wchan < p.N;

  auto load_tiles = [&](int k0) {
    if constexpr (AF32) {
      const float* x = static_cast<const float*>(p.a);
      const int c = tid & 15;
#pragma unroll
      for (int i = 0; i < XR; ++i)
        xr[i] = xrow[i] >= 0 ? *reinterpret_cast<const uint4*>(x + xrow[i] * p.lda + k0 + 4 * c) : zero4();
    } else {
      const uint16_t* x = static_cast<const uint16_t*>(p.a);
      const int c = tid & 7;
#pragma unroll
      for (int i = 0; i < XR; ++i)
        xr[i] = xrow[i] >= 0 ? *reinterpret_cast<const uint4*>(x + xrow[i] * p.lda + k0 + 8 * c) : zero4();
    }
    const size_t n = (size_t)wchan;
    if constexpr (FP8) {
      const uint8_t* src = wc + (size_t)n * K + k0 + 32 * w_half;
      wr[0] = w_ok ? *reinterpret_cast<const uint4*>(src) : zero4();
      wr[1] = w_ok ? *reinterpret_cast<const uint4*>(src + 16) : zero4();
    } else {
      const uint8_t* src = wc + (size_t)n * (K / 2) + k0 / 2 + 16 * w_half;
      wr[0] = w_ok ? *reinterpret_cast<const uint4*>(src) : zero4();
      wsb = w_ok ? ws_h[n * (K / p.g) + (k0 + 32 * w_half) / p.g] : (uint16_t)0;
    }
  };

  auto store_tiles = [&](int buf) {
    uint16_t* Xs = smem + buf * STAGE;
    uint16_t* Ws = Xs + BM * LDK;
    if constexpr (AF32) {
      const int c = tid & 15;
#pragma unroll
      for (int i = 0; i < XR; ++i) {
        const int r = (tid >> 4) + 16 * i;
        const float4 v = __builtin_bit_cast(float4, xr[i]);
        *reinterpret_cast<uint2*>(&Xs[r * LDK + 4 * c]) =
            make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
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
      const uint32_t wv[8] = {wr[0].x, wr[0].y, wr[0].z, wr[0].w, wr[1].x, wr[1].y, wr[1].z, wr[1].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint2 lo = dq_fp8x4(wv[2 * q]), hi = dq_fp8x4(wv[2 * q + 1]);
        dst[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    } else {
      const auto wsc = W4<WF>::scale(wsb);
      dst[0] = W4<WF>::dq(wr[0].x, wsc);
      dst[1] = W4<WF>::dq(wr[0].y, wsc);
      dst[2] = W4<WF>::dq(wr[0].z, wsc);
      dst[3] = W4<WF>::dq(wr[0].w, wsc);
    }
  };

  f32x16 acc[2][TM];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  auto compute = [&](int buf) {
    const uint16_t* Xs = smem + buf * STAGE;
    const uint16_t* Ws = Xs + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[2], b[TM];
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        a[tn] = *reinterpret_cast<const bf16x8*>(&Ws[(wn * 64 + tn * 32 + l32) * LDK + kk * 16 + 8 * g2]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        b[tm] = *reinterpret_cast<const bf16x8*>(&Xs[(wm * (BM / 2) + tm * 32 + l32) * LDK + kk * 16 + 8 * g2]);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[tn][tm] = mfma32(a[tn], b[tm], acc[tn][tm]);
    }
  };

  const int nk = K / BK;
  if constexpr (NBUF == 2) {
    load_tiles(0);
    store_tiles(0);
    if (nk > 1) load_tiles(BK);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
      compute(s & 1);
      if (s + 1 < nk) store_tiles((s + 1) & 1);
      if (s + 2 < nk) load_tiles((s + 2) * BK);
      __syncthreads();
    }
  } else {
    load_tiles(0);
    for (int s = 0; s < nk; ++s) {
      if (s > 0) __syncthreads();
      store_tiles(0);
      __syncthreads();
      if (s + 1 < nk) load_tiles((s + 1) * BK);
      compute(0);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  uint32_t swg[2][TM][8];  // EPI_ROT_SWIGLU: bf16 pairs of this lane's outputs
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const int nb = w_chan(wn * 64 + tn * 32);  // first channel of this 32-group
    const bool n_ok = nb < p.N;
    float sc[16];
    if constexpr (FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (n_ok) v = *reinterpret_cast<const float4*>(ws_f + nb + 8 * q + 4 * g2);
        sc[4 * q] = v.x;
        sc[4 * q + 1] = v.y;
        sc[4 * q + 2] = v.z;
        sc[4 * q + 3] = v.w;
      }
    }
    bf16x8 ra[2];
    if constexpr (epi_rotates(EPI)) {
      // A operand: R rows j = l32; items follow the accumulator row order
      // i(t, p) = 16t + 8(p/4) + 4g2 + p%4.
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint2 lo = make_uint2(0u, 0u), hi = make_uint2(0u, 0u);
        if (n_ok) {
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
        }
        ra[t] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      f32x16 z = acc[tn][tm];
      if constexpr (FP8) {
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] *= sc[r];
      }
      f32x16 o;
      if constexpr (epi_rotates(EPI)) {
        bf16x8 zb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          zb[t] = as_bf16x8(make_uint4(pack_bf16x2(z[8 * t], z[8 * t + 1]), pack_bf16x2(z[8 * t + 2], z[8 * t + 3]),
                                       pack_bf16x2(z[8 * t + 4], z[8 * t + 5]), pack_bf16x2(z[8 * t + 6], z[8 * t + 7])));
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = 0.0f;
        o = mfma32(ra[0], zb[0], o);
        o = mfma32(ra[1], zb[1], o);
      } else {
        o = z;
      }
      const int ml = wm * (BM / 2) + tm * 32 + l32;
      const bool m_ok = n_ok && ml < nrows;
      const long orow = (long)(pos0 + ml);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = pack_bf16x2(o[4 * q], o[4 * q + 1]);
        const uint32_t hi = pack_bf16x2(o[4 * q + 2], o[4 * q + 3]);
        if constexpr (EPI == EPI_ROT_SWIGLU) {
          swg[tn][tm][2 * q] = lo;
          swg[tn][tm][2 * q + 1] = hi;
        }
        if (m_ok) {
          const size_t off = (size_t)orow * p.ldo + nb + 8 * q + 4 * g2;
          if constexpr (OUTF32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off) =
                make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
          } else {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) = make_uint2(lo, hi);
          }
        }
      }
    }
  }

  if constexpr (EPI == EPI_ROT_SWIGLU) {
    // up waves (wn = 1) hand their bf16 outputs to the gate waves (wn = 0)
    // holding the same (token, channel) slots; the tiles are free now.
    static_assert(2 * 2 * TM * 64 * 8 * 4 <= NBUF * STAGE * 2, "exchange buffer");
    uint32_t* xb = reinterpret_cast<uint32_t*>(smem);
    if (wn == 1) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int v = 0; v < 8; ++v) xb[(((wm * 2 + tn) * TM + tm) * 8 + v) * 64 + lane] = swg[tn][tm][v];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const int cb = blockIdx.x * (BN / 2) + tn * 32;  // gate channel base = act column base
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int ml = wm * (BM / 2) + tm * 32 + l32;
          if (cb >= p.half_n || ml >= nrows) continue;
          const long orow = (long)(pos0 + ml);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float av[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t gw = swg[tn][tm][2 * q + h];
              const uint32_t uw = xb[(((wm * 2 + tn) * TM + tm) * 8 + 2 * q + h) * 64 + lane];
#pragma unroll
              for (int s = 0; s < 2; ++s) {
                const float gv = bf16_to_f32((uint16_t)(gw >> (16 * s)));
                const float uv = bf16_to_f32((uint16_t)(uw >> (16 * s)));
                av[2 * h + s] = gv / (1.0f + __expf(-gv)) * uv;
              }
            }
            *reinterpret_cast<uint2*>(p.act + (size_t)orow * p.ldact + cb + 8 * q + 4 * g2) =
                make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
          }
        }
      }
    }
  }
}

}  // namespace oft
