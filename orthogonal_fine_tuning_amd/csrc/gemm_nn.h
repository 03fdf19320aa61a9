// Generic backward-type dequant GEMM:  C^T[k][m] = sum_n W[n][k] B'[m][n]
// where the contraction runs over the weight's rows n and B' is built from
// bf16 source rows by a prologue:
//   PRO_ROT  : B'_blk = src_blk R_j (computed as R_j^T src^T on the matrix
//              cores; FP8 also multiplies channel n by s_n), rounded to bf16;
//   PRO_NONE : B' = src.
// The weight tile [64 n x 128 k] (INT4 or FP8 codes, or bf16 values) is
// dequantised in registers and stored to LDS with k contiguous (16-byte
// stores; 256-byte rows, chunk c of row n at c ^ 4 (n % 4)); the matrix-core
// operand, which must run along the contraction n, is read with the gfx950
// LDS transpose load (ds_read_b64_tr_b16: within each 16-lane group, lane i
// receives element i % 4 of the 8-byte chunks loaded by lanes 4e + i / 4,
// e = 0..3; pointing lane r at row n0 + r / 4, column k0 + 4 (r % 4) gives
// lane i the four values W[n0 .. n0+3][k0 + i]).  Two LDS buffers, registers
// one step ahead, one barrier per step as in gemm_nt.h.  Rows are dense
// tokens or grouped expert positions exactly as in gemm_nt.h (kslots > 0
// gathers src row perm[pos] / kslots).
// Epilogues:
//   EPI_STORE      : store C rows (bf16 or fp32);
//   EPI_SWIGLU_BWD : C = d act (before the combine weight) for the down
//                    projection; with h = (gate, up) from the saved
//                    activations and w the pair's combine weight:
//                      dw partial  = sum_k C * silu(gate) * up (this k tile),
//                      d gate      = w C up sig (1 + gate (1 - sig)),
//                      d up        = w C silu(gate),
//                    written to dH rows (gate half at k, up half at I + k).
#pragma once

#include <type_traits>

#include "oft_device.h"

namespace oft {

enum : int { PRO_ROT = 0, PRO_NONE = 1 };
enum : int { EPI_STORE = 0, EPI_SWIGLU_BWD = 1 };

struct NnArgs {
  const uint16_t* src;
  long lds;
  const uint8_t* wc;
  const void* ws;
  long wc_e, ws_e;
  const uint16_t* rops;
  long rops_e;
  void* out;
  long ldo;
  int M, K, N, g;  // K: output columns (weight columns), N: contraction (weight rows)
  const int* tiles;
  const int* ntiles;
  const int* offsets;
  const int* perm;
  int kslots;
  // EPI_SWIGLU_BWD
  const uint16_t* hsave;  // [P, 2I]
  long ldh;
  const float* topk_w;    // [P] by pair id
  float* dw_part;         // [K / 128][P] by position
  long P;
  // contraction split (few-token layers): workgroup z covers weight rows
  // [z * nsplit_len, (z + 1) * nsplit_len) and stores fp32 partials to
  // part[z][M][K]; nsplit_len == 0 means no split
  int nsplit_len;
  float* part;
};

namespace nn {
constexpr int BKO = 128;       // output columns per tile
constexpr int BNS = 64;        // contraction step
constexpr int LDN = BNS + 8;   // B' rows (n contiguous)
constexpr int LDW = BKO;       // weight rows (k contiguous), 256 bytes; 16-byte chunk
                               // c of row n stored at c ^ 4 (n % 4)
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ uint2 ds_read_tr16(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  return __builtin_bit_cast(uint2, v);
}
}  // namespace nn

template <int BM, bool OUTF32, int WF, int B, int PRO, int EPI, bool GROUPED, int NBUF = 2>
__global__ __launch_bounds__(256, (BM == 256 && NBUF == 2) ? 1 : 2) void gemm_nn_kernel(NnArgs p) {
  using namespace nn;
  static_assert(BM == 128 || BM == 256, "tile");
  static_assert(!wf_tiled(WF), "row-major weights only");
  constexpr bool FP8 = WF == WF_FP8;
  constexpr bool W16 = WF == WF_BF16;  // bf16 weights: plain copies into the tile
  constexpr int TM = BM / 64;   // 32-token tiles per wave (main product)
  constexpr int PM = BM / 128;  // 32-token tiles each wave prepares in the prologue
  constexpr int WSZ = BNS * LDW;        // weight tile [n][k]
  constexpr int STAGE = WSZ + BM * LDN;  // + B' tile [m][n]
  static_assert(NBUF == 1 || NBUF == 2, "buffers");
  __shared__ __attribute__((aligned(16))) uint16_t smem[NBUF * STAGE];
  __shared__ float dwred[EPI == EPI_SWIGLU_BWD ? 2 * BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int wk = wave >> 1, wm = wave & 1;
  const int K = p.K, N = p.N;
  int e = 0, pos0, nrows, cx = blockIdx.x;
  if constexpr (GROUPED) {
    int t;
    if (!grouped_tile(*p.ntiles, cx, t)) return;
    e = p.tiles[2 * t];
    const int r0 = p.tiles[2 * t + 1];
    pos0 = p.offsets[e] + r0;
    nrows = min(BM, p.offsets[e + 1] - pos0);
  } else {
    pos0 = blockIdx.y * BM;
    nrows = min(BM, p.M - pos0);
  }
  const int k0 = cx * BKO;
  const uint8_t* wc = p.wc + (size_t)e * p.wc_e;
  const uint16_t* rops = p.rops + (size_t)e * p.rops_e;
  const float* ws_f = static_cast<const float*>(p.ws);
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws) + (size_t)e * p.ws_e;

  // W tile: thread owns row n0 + wrow, columns k0 + 32*wq + 0..31
  const int wrow = tid >> 2, wq = tid & 3;
  const bool k_ok = (k0 + 32 * wq) < K;
  uint4 wr[W16 ? 4 : FP8 ? 2 : 1];
  uint16_t wsb = 0;  // INT4: fp16 scale bits of the prefetched weight row

  // source rows this wave feeds to the prologue
  long srow[PM];
#pragma unroll
  for (int i = 0; i < PM; ++i) {
    const int ml = (PM * wave + i) * 32 + l32;
    long r = -1;
    if (ml < nrows) {
      r = pos0 + ml;
      if constexpr (GROUPED) {
        if (p.kslots > 0) r = p.perm[pos0 + ml] / p.kslots;
      }
    }
    srow[i] = r;
  }
  uint4 sf[PM][2][2];  // [i][32-channel group][t] source operand fragments
  uint4 rtf[2][2];     // [32-channel group][t] R^T operand fragments
  float4 scf[2][4];    // FP8 channel scales, accumulator order

  auto prefetch = [&](int n0) {
    {
      const int n = n0 + wrow;
      const bool ok = k_ok && n < N;
      if constexpr (W16) {
        const uint8_t* src = wc + ((size_t)n * K + k0 + 32 * wq) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[i] = ok ? *reinterpret_cast<const uint4*>(src + 16 * i) : zero4();
      } else if constexpr (FP8) {
        const uint8_t* src = wc + (size_t)n * K + k0 + 32 * wq;
        wr[0] = ok ? *reinterpret_cast<const uint4*>(src) : zero4();
        wr[1] = ok ? *reinterpret_cast<const uint4*>(src + 16) : zero4();
      } else {
        wr[0] = ok ? *reinterpret_cast<const uint4*>(wc + (size_t)n * (K / 2) + (k0 + 32 * wq) / 2) : zero4();
        wsb = ok ? ws_h[(size_t)n * (K / p.g) + (k0 + 32 * wq) / p.g] : (uint16_t)0;
      }
    }
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const int nb = n0 + 32 * grp;
      const bool gok = nb < N;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (PRO == PRO_ROT) {
          uint4 v = zero4();
          if (gok) {
            if constexpr (B == 32) {
              v = *reinterpret_cast<const uint4*>(rops + (size_t)(nb / 32) * 2048 + 1024 + l32 * 32 + 16 * t + 8 * g2);
            } else {
              if ((l32 >> 4) == t)
                v = *reinterpret_cast<const uint4*>(rops + (size_t)(nb / 16 + t) * 512 + 256 + (l32 & 15) * 16 + 8 * g2);
            }
          }
          rtf[grp][t] = v;
        }
#pragma unroll
        for (int i = 0; i < PM; ++i)
          sf[i][grp][t] = (gok && srow[i] >= 0)
                              ? *reinterpret_cast<const uint4*>(p.src + srow[i] * p.lds + nb + 16 * t + 8 * g2)
                              : zero4();
      }
      if constexpr (FP8 && PRO == PRO_ROT) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          scf[grp][q] = gok ? *reinterpret_cast<const float4*>(ws_f + nb + 8 * q + 4 * g2)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };

  auto stage = [&](int buf) {
    uint16_t* Ws = smem + buf * STAGE;
    uint16_t* Bs = Ws + WSZ;
    // W tile -> LDS: this thread's chunks 4 wq + u (u = 0..3) of row wrow,
    // chunk c stored at c ^ 4 (wrow % 4); the i-th store writes u = (i + wq)
    // % 4 (the order measured free of bank conflicts; the plain order ran
    // at less than half the write rate)
    uint16_t* wrow_p = Ws + wrow * LDW;
    const int wx = 4 * (wrow & 3);
    auto put = [&](int i, uint4 v) {
      const int c = (4 * wq + ((i + wq) & 3)) ^ wx;
      *reinterpret_cast<uint4*>(wrow_p + 8 * c) = v;
    };
    // rotate four per-lane units by wq: out[i] = in[(i + wq) % 4]
    auto rot4 = [&](auto* v) {
      auto t1 = v[0];
      if (wq & 1) { t1 = v[0]; v[0] = v[1]; v[1] = v[2]; v[2] = v[3]; v[3] = t1; }
      if (wq & 2) { t1 = v[0]; v[0] = v[2]; v[2] = t1; t1 = v[1]; v[1] = v[3]; v[3] = t1; }
    };
    if constexpr (W16) {
      uint4 v[4] = {wr[0], wr[1], wr[2], wr[3]};
      rot4(v);
#pragma unroll
      for (int i = 0; i < 4; ++i) put(i, v[i]);
    } else if constexpr (FP8) {
      uint2 v[4] = {make_uint2(wr[0].x, wr[0].y), make_uint2(wr[0].z, wr[0].w), make_uint2(wr[1].x, wr[1].y),
                    make_uint2(wr[1].z, wr[1].w)};
      rot4(v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 lo = dq_fp8x4(v[i].x), hi = dq_fp8x4(v[i].y);
        put(i, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    } else {
      const auto wsc = W4<WF>::scale(wsb);
      uint32_t v[4] = {wr[0].x, wr[0].y, wr[0].z, wr[0].w};
      rot4(v);
#pragma unroll
      for (int i = 0; i < 4; ++i) put(i, W4<WF>::dq(v[i], wsc));
    }
    // prologue -> Bs[m][n]
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
#pragma unroll
      for (int i = 0; i < PM; ++i) {
        const int ml = (PM * wave + i) * 32 + l32;
        if constexpr (PRO == PRO_NONE) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            *reinterpret_cast<uint4*>(&Bs[ml * LDN + 32 * grp + 16 * t + 8 * g2]) = sf[i][grp][t];
        } else {
          f32x16 o;
#pragma unroll
          for (int r = 0; r < 16; ++r) o[r] = 0.0f;
          o = mfma32(as_bf16x8(rtf[grp][0]), as_bf16x8(sf[i][grp][0]), o);
          o = mfma32(as_bf16x8(rtf[grp][1]), as_bf16x8(sf[i][grp][1]), o);
          if constexpr (FP8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              o[4 * q] *= scf[grp][q].x;
              o[4 * q + 1] *= scf[grp][q].y;
              o[4 * q + 2] *= scf[grp][q].z;
              o[4 * q + 3] *= scf[grp][q].w;
            }
          }
          // Lane (m, g2) holds channels 8q + 4g2 + 0..3 in registers 4q..4q+3.
          // Swapping one 4-channel run with lane m + 32(1 - g2) leaves lane g2
          // with channels 16h + 8g2 + 0..7 of the pair q = 2h, 2h + 1.
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint2 p0 = make_uint2(pack_bf16x2(o[8 * h], o[8 * h + 1]), pack_bf16x2(o[8 * h + 2], o[8 * h + 3]));
            const uint2 p1 = make_uint2(pack_bf16x2(o[8 * h + 4], o[8 * h + 5]), pack_bf16x2(o[8 * h + 6], o[8 * h + 7]));
            const uint2 snd = g2 ? p0 : p1;
            uint2 rcv;
            rcv.x = (uint32_t)__shfl_xor((int)snd.x, 32);
            rcv.y = (uint32_t)__shfl_xor((int)snd.y, 32);
            const uint4 v = g2 ? make_uint4(rcv.x, rcv.y, p1.x, p1.y) : make_uint4(p0.x, p0.y, rcv.x, rcv.y);
            *reinterpret_cast<uint4*>(&Bs[ml * LDN + 32 * grp + 16 * h + 8 * g2]) = v;
          }
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

  // A operand (W^T rows k, contraction n) through the LDS transpose load
  const int G = lane >> 4, li = lane & 15;
  // TMV (a std::integral_constant): this wave's 32-row tiles that hold rows
  // (grouped tiles past an expert's last row skip the rest)
  auto compute = [&](int buf, auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    if constexpr (TMV == 0) return;
    const uint16_t* Ws = smem + buf * STAGE;
    const uint16_t* Bs = Ws + WSZ;
#pragma unroll
    for (int kk = 0; kk < BNS / 16; ++kk) {
      bf16x8 a[2], b[TM];
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        const int kcol = wk * 64 + tk * 32 + 16 * (G & 1) + 4 * (li & 3);
        const int nrow = kk * 16 + 8 * (G >> 1) + (li >> 2);
        const int off = nrow * LDW + 8 * ((kcol >> 3) ^ (4 * (nrow & 3))) + (kcol & 7);
        const uint2 lo = ds_read_tr16(&Ws[off]);
        const uint2 hi = ds_read_tr16(&Ws[off + 4 * LDW]);
        a[tk] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm)
        b[tm] = *reinterpret_cast<const bf16x8*>(&Bs[(wm * (BM / 2) + tm * 32 + l32) * LDN + kk * 16 + 8 * g2]);
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
#pragma unroll
        for (int tm = 0; tm < TMV; ++tm) acc[tk][tm] = mfma32(a[tk], b[tm], acc[tk][tm]);
    }
  };

  const int nbeg = p.nsplit_len > 0 ? blockIdx.z * p.nsplit_len : 0;
  const int nend = p.nsplit_len > 0 ? min(N, nbeg + p.nsplit_len) : N;
  const int ns = (nend - nbeg + BNS - 1) / BNS;
  // every wave stages its share and takes every barrier, whatever its TMV
  auto run = [&](auto tmv_c) {
    if constexpr (NBUF == 2) {
      if (ns > 0) {
        prefetch(nbeg);
        stage(0);
        if (ns > 1) prefetch(nbeg + BNS);
      }
      __syncthreads();
      for (int s = 0; s < ns; ++s) {
        compute(s & 1, tmv_c);
        if (s + 1 < ns) stage((s + 1) & 1);
        if (s + 2 < ns) prefetch(nbeg + (s + 2) * BNS);
        __syncthreads();
      }
    } else {
      if (ns > 0) prefetch(nbeg);
      for (int s = 0; s < ns; ++s) {
        if (s > 0) __syncthreads();
        stage(0);
        __syncthreads();
        if (s + 1 < ns) prefetch(nbeg + (s + 1) * BNS);
        compute(0, tmv_c);
      }
      __syncthreads();
    }
  };
  if constexpr (GROUPED) {
    static_assert(TM == 2, "grouped tiles: 128 rows");
    const int rows_w = nrows - wm * (BM / 2);  // rows of this wave's 64 (uniform)
    if (rows_w > 32)
      run(std::integral_constant<int, 2>{});
    else if (rows_w > 0)
      run(std::integral_constant<int, 1>{});
    else
      run(std::integral_constant<int, 0>{});
  } else {
    run(std::integral_constant<int, TM>{});
  }

  // ------------------------------------------------------------ epilogue
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int tk = 0; tk < 2; ++tk) {
      const int kb = k0 + wk * 64 + tk * 32;
      if (kb >= K) continue;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int ml = wm * (BM / 2) + tm * 32 + l32;
        if (ml >= nrows) continue;
        const long orow = (long)(pos0 + ml);
        const f32x16& o = acc[tk][tm];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const size_t off = (size_t)orow * p.ldo + kb + 8 * q + 4 * g2;
          if (p.nsplit_len > 0) {
            *reinterpret_cast<float4*>(p.part + (size_t)blockIdx.z * p.M * p.ldo + off) =
                make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
          } else if constexpr (OUTF32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off) =
                make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
          } else {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) =
                make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
          }
        }
      }
    }
  } else {
    // SwiGLU backward; out = dH [P, 2I] with ldo, K = I
    float dwp[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) dwp[tm] = 0.0f;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int ml = wm * (BM / 2) + tm * 32 + l32;
      const bool m_ok = ml < nrows;
      const long pos = (long)(pos0 + ml);
      const float wgt = m_ok ? p.topk_w[p.perm[pos]] : 0.0f;
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        const int kb = k0 + wk * 64 + tk * 32;
        if (kb >= K || !m_ok) continue;
        const f32x16& o = acc[tk][tm];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = kb + 8 * q + 4 * g2;
          const uint2 hg = *reinterpret_cast<const uint2*>(p.hsave + pos * p.ldh + col);
          const uint2 hu = *reinterpret_cast<const uint2*>(p.hsave + pos * p.ldh + K + col);
          const uint32_t gw[2] = {hg.x, hg.y}, uw[2] = {hu.x, hu.y};
          float dg[4], du[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float gv = bf16_to_f32((uint16_t)(gw[s >> 1] >> (16 * (s & 1))));
            const float uv = bf16_to_f32((uint16_t)(uw[s >> 1] >> (16 * (s & 1))));
            const float sg = 1.0f / (1.0f + __expf(-gv));
            const float silu = gv * sg;
            const float da_u = o[4 * q + s];
            dwp[tm] += da_u * silu * uv;
            const float da = wgt * da_u;
            dg[s] = da * uv * sg * (1.0f + gv * (1.0f - sg));
            du[s] = da * silu;
          }
          uint16_t* dh = static_cast<uint16_t*>(p.out) + pos * p.ldo;
          *reinterpret_cast<uint2*>(dh + col) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *reinterpret_cast<uint2*>(dh + K + col) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
        }
      }
    }
    // per-position partial over this k tile: lanes g2 = 0/1, then waves wk = 0/1
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) dwp[tm] += __shfl_xor(dwp[tm], 32);
    if (wk == 1 && g2 == 0) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) dwred[wm * (BM / 2) + tm * 32 + l32] = dwp[tm];
    }
    __syncthreads();
    if (wk == 0 && g2 == 0) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int ml = wm * (BM / 2) + tm * 32 + l32;
        if (ml < nrows) p.dw_part[(size_t)cx * p.P + pos0 + ml] = dwp[tm] + dwred[ml];
      }
    }
  }
}

}  // namespace oft
