// 4-bit dequant GEMM on 128-row tiles with half-line weight copies.
//
// Same product, tile (256 channels x 128 rows, grouped or dense), wave
// layout (8 waves of 32 channels over every row, each code row dequantised
// once), epilogues and results as gemm_nt_dma_kernel on INT4 / FP4 weights,
// with a different weight stream.  There each 64-wide K step copies 32 bytes
// of every weight row, 32 rows per copy instruction, so each 128-byte line
// of codes is requested by four instructions in four steps.  Here a weight
// stage holds two steps (64 bytes of every row: 16 rows per instruction,
// each line requested twice) and is copied one stage (two steps) ahead; the
// activation ring keeps one step of lookahead in two stages, so that the
// workgroup still fits twice per CU (68 KB):
//   activations  two stages of 128 rows x 128 B, chunk c of row r at
//                c ^ swz_x(r)
//   weights      two stages of 256 rows x 64 B (chunk c of row r at
//                c ^ swz_w8(r), the FP8 layout) followed by the two steps'
//                scale words (256 rows x 4 B each)
// Copies are issued activations first, then (at even steps) the next
// weight stage, so that waiting for step s's activations leaves that
// weight stage in flight: the weights get two steps of latency, the
// activations (mostly L2 hits) one.
//
// Tiled INT4 storage (WF_INT4T, see oft_formats.h): a stage is one tile
// column of each 64-row block, so each wave's 32 rows read 2 KB of codes and
// 256/g bytes a row of scales, each contiguous in memory (row-major: 64-byte
// pieces 8 KB apart and one 4-byte scale word per row and step).  The LDS
// holds the stage's scales as the tiles do, 256/g bytes a row (4-byte slots
// for g = 64 and 128).
#pragma once

#include "gemm_nt_dma.h"

namespace oft {

namespace nth {
constexpr int NTHR = 512;
constexpr int BN = 256, BM = 128;
constexpr int XROW = 128;             // activation bytes per row and step
constexpr int XB = BM * XROW;         // 16 KB per activation stage
constexpr int WROW = 64;              // code bytes per row and weight stage (two steps)
constexpr int WCB = BN * WROW;        // 16 KB
constexpr int WSB = 2 * BN * 4;       // the two steps' scale words
constexpr int WB = WCB + WSB;
constexpr int SMEM = 2 * XB + 2 * WB;  // 68 KB: two workgroups per CU
static_assert(2 * SMEM <= 160 * 1024, "LDS");
}  // namespace nth

template <int WF, int B, int EPI, bool GROUPED>
__global__ __launch_bounds__(nth::NTHR, 2) void gemm_nt_hl_kernel(NtArgs p) {
  using namespace ntd;
  static_assert(wf_4bit(WF), "4-bit weights");
  static_assert(EPI == EPI_ROT || EPI == EPI_PLAIN || epi_swiglu(EPI) || EPI == EPI_BASE, "epilogue");
  constexpr bool SWI = epi_swiglu(EPI);
  constexpr int BN = nth::BN, BM = nth::BM, XB = nth::XB, XROW = nth::XROW, WB = nth::WB, WCB = nth::WCB;
  constexpr int TM = BM / 32;
  constexpr bool TILED = wf_tiled(WF);
  constexpr int XI = 2;   // activation copies per wave and step (16 rows)
  // copies per wave and weight stage: 2 of codes, then 2 of scale words
  // (row-major) or 1 of the stage's scale slots (tiled)
  constexpr int WC = TILED ? 3 : 4;
  __shared__ __attribute__((aligned(16))) uint8_t xs[2 * XB];
  __shared__ __attribute__((aligned(16))) uint8_t wsm[2 * WB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;

  // ---- tile
  int e = 0, pos0, nrows, cx = blockIdx.x;
  if constexpr (GROUPED) {
    int t;
    if (!grouped_tile(*p.ntiles, cx, t)) return;
    e = p.tiles[2 * t];
    pos0 = p.offsets[e] + p.tiles[2 * t + 1];
    nrows = min(BM, p.offsets[e + 1] - pos0);
  } else {
    pos0 = blockIdx.y * BM;
    nrows = min(BM, p.M - pos0);
  }
  const uint8_t* wc = p.wc + (size_t)e * p.wc_e;
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws) + (size_t)e * p.ws_e;
  const uint16_t* rops = nt_rops(p) + (size_t)e * p.rops_e;
  const int cbase = SWI ? cx * (BN / 2) : cx * BN;
  auto chan = [&](int rw) -> int {
    if constexpr (SWI) {
      const int c = cbase + (rw & (BN / 2 - 1));
      return c < p.half_n ? (rw < BN / 2 ? c : p.half_n + c) : -1;
    } else {
      return cbase + rw < p.N ? cbase + rw : -1;
    }
  };
  auto crow = [&](int rw) { const int c = chan(rw); return c >= 0 ? c - cbase : 0; };
  const int nk = K / 64;   // steps (even)
  const int nu = nk / 2;   // weight stages
  const int kg = K / p.g;
  const int gs = p.g == 32 ? 1 : p.g == 64 ? 0 : -1;  // log2(64 / g)

  // ---- copy sources
  // activations: rows 16 wave + 8 i + lane / 8; the copies of rows past the
  // tile's end are skipped (their products are never stored)
  const uint8_t* xbase = static_cast<const uint8_t*>(p.a) + (size_t)pos0 * p.lda * 2;
  uint32_t xoff[XI];
  const uint8_t* xptr[GROUPED ? XI : 1];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = 16 * wave + 8 * i + (lane >> 3);
    const int rr = r < nrows ? r : 0;
    const int chunk = 16 * ((lane & 7) ^ swz_x(r));
    xoff[i] = (uint32_t)(rr * p.lda * 2 + chunk);
    if constexpr (GROUPED) {
      const long src = p.kslots > 0 ? (long)(p.perm[pos0 + rr] / p.kslots) : (long)(pos0 + rr);
      xptr[i] = static_cast<const uint8_t*>(p.a) + src * p.lda * 2 + chunk;
    }
  }
  int xc = 0;
#pragma unroll
  for (int i = 0; i < XI; ++i) xc += 16 * wave + 8 * i < nrows ? 1 : 0;
  const uint32_t x_lds = lds_addr(xs) + (uint32_t)(2048 * wave);
  // weight codes: rows 32 wave + 16 i + lane / 4, 16-byte chunk lane % 4 of
  // the stage's 64 bytes
  // (tiled: cbase is a multiple of 64, so its block starts at the same
  // byte as its row-major row, and t4_code_off of the row relative to cbase
  // is the offset from there)
  const uint8_t* wbase = wc + (size_t)cbase * (K / 2);
  uint32_t woff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rw = 32 * wave + 16 * i + (lane >> 2);
    const int cb = 16 * ((lane & 3) ^ swz_w8(rw));
    woff[i] = TILED ? t4_code_off(crow(rw), cb, K) : (uint32_t)(crow(rw) * (K / 2) + cb);
  }
  constexpr int WSTRIDE = TILED ? T4_TILE_BYTES : nth::WROW;  // bytes from one weight stage to the next
  const uint32_t w_lds = lds_addr(wsm) + (uint32_t)(2048 * wave);
  // scale words: lanes 0..31 copy the 4-byte word holding step s's scale(s)
  // of row 32 wave + lane
  const uint32_t sbase = (uint32_t)((cbase + crow(32 * wave + l32)) * kg);
  const uint32_t s_lds = lds_addr(wsm) + (uint32_t)(WCB + 32 * wave * 4);
  // tiled scales: bytes a row in the LDS (8 for g = 32, else a 4-byte slot
  // per row), the wave's copy (g = 32: lane 2 r + d takes 4-byte word d of
  // row 32 wave + r; else lanes 0..31 one row each) and its source offset
  // from the block of cbase, stage 0; stage u adds u * 16384 / g
  const int srow = p.g == 32 ? 8 : 4;
  const int s_rw = p.g == 32 ? 32 * wave + (lane >> 1) : 32 * wave + l32;
  const uint32_t st_off = TILED ? t4_scale_off(crow(s_rw), 0, K, p.g) + (p.g == 32 ? 4u * (lane & 1) : 0u) : 0u;
  const uint32_t st_lds = lds_addr(wsm) + (uint32_t)(WCB + 32 * wave * srow);
  const uint32_t st_stride = (uint32_t)(16384 / p.g);
  const uint8_t* ws_b = reinterpret_cast<const uint8_t*>(ws_h) + (size_t)cbase * kg * 2;
  auto sstep = [&](int s) { return gs >= 0 ? s << gs : s >> 1; };  // first scale of step s: 64 s / g

  auto issue_x = [&](int s, int c) {
    if (c >= xc) return;
    const uint32_t dst = x_lds + (uint32_t)((s & 1) * XB + c * 1024);
    if constexpr (GROUPED)
      copy16v(dst, xptr[c] + (size_t)s * XROW);
    else
      copy16(dst, xbase + (size_t)s * XROW, xoff[c]);
  };
  // copy c (0..3) of weight stage u: codes (c = 0, 1), scale words of its
  // steps (c = 2, 3)
  auto issue_w = [&](int u, int c) {
    const uint32_t b = (uint32_t)((u & 1) * WB);
    if (c < 2) {
      copy16(w_lds + b + 1024 * c, wbase + (size_t)u * WSTRIDE, woff[c]);
    } else if constexpr (TILED) {
      const uint8_t* src = ws_b + (size_t)u * st_stride;
      if (p.g == 32)
        copy4(st_lds + b, src, st_off);
      else if (lane < 32) {
        if (p.g == 64)
          copy4(st_lds + b, src, st_off);
        else
          copy2(st_lds + b, src, st_off);
      }
    } else {
      const int s = 2 * u + (c - 2);
      if (lane < 32) copy4(s_lds + b + (uint32_t)((c - 2) * BN * 4), ws_h, ((sbase + (uint32_t)sstep(s)) * 2u) & ~3u);
    }
  };

  // ---- operand reads
  const int rw = 32 * wave + l32;  // this lane's operand row
  const uint32_t wrd = (uint32_t)(rw * nth::WROW);
  const int wsw = swz_w8(rw);
  const uint32_t srd = (uint32_t)((cbase + crow(rw)) * kg);  // scale index of row rw at k = 0
  uint32_t xrd[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) xrd[tm] = (uint32_t)((32 * tm + l32) * XROW);
  const int xsw = swz_x(l32);
  const int xg = 4 * g2;

  f32x16 acc[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;

  // step s: this lane's in-features 64 s + 32 g2 .. + 31 are 16-byte chunk
  // 2 t + g2 of the stage row (t = s % 2); MFMA group kk takes word kk.
  // The next copies are spread over the groups: activations after group 0,
  // the weight stage (even steps) after groups 1..3.
  auto compute = [&](int s, auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    const int t = s & 1, u = s >> 1;
    const bool nx = s + 1 < nk;
    const bool nw = t == 0 && u + 1 < nu;
    if constexpr (TMV == 0) {
      if (nx)
        for (int c = 0; c < XI; ++c) issue_x(s + 1, c);
      if (nw)
        for (int c = 0; c < WC; ++c) issue_w(u + 1, c);
      return;
    }
    const uint8_t* X = xs + (s & 1) * XB;
    const uint8_t* W = wsm + (u & 1) * WB;
    const uint4 c4 = *reinterpret_cast<const uint4*>(W + wrd + 16 * ((2 * t + g2) ^ wsw));
    const uint32_t cw[4] = {c4.x, c4.y, c4.z, c4.w};
    uint32_t word, half;
    if constexpr (TILED) {
      word = *reinterpret_cast<const uint32_t*>(W + WCB + rw * srow + (gs == 1 ? 4 * t : 0));
      half = gs == 1 ? g2 : gs == 0 ? t : 0;
    } else {
      word = *reinterpret_cast<const uint32_t*>(W + WCB + t * BN * 4 + rw * 4);
      half = (srd + (uint32_t)(gs == 1 ? 2 * s + g2 : gs == 0 ? s : s >> 1)) & 1;
    }
    const typename W4<WF>::S sc = W4<WF>::scale((uint16_t)(word >> (16 * half)));
    auto load_b = [&](int kk, bf16x8* b) {
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) b[tm] = *reinterpret_cast<const bf16x8*>(X + xrd[tm] + 16 * ((xg + kk) ^ xsw));
    };
    bf16x8 aq[2], bq[2][TMV];
    load_b(0, bq[0]);
    aq[0] = as_bf16x8(W4<WF>::dq(cw[0], sc));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < 4) load_b(kk + 1, bq[c ^ 1]);
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) acc[tm] = mfma32(aq[c], bq[c][tm], acc[tm]);
      if (kk == 0 && nx) {
#pragma unroll
        for (int cc = 0; cc < XI; ++cc) issue_x(s + 1, cc);
      }
      if (kk >= 1 && nw) {
        issue_w(u + 1, kk - 1);
        if (kk == 3 && WC > 3) issue_w(u + 1, 3);
      }
      if (kk + 1 < 4) aq[c ^ 1] = as_bf16x8(W4<WF>::dq(cw[kk + 1], sc));
    }
  };

  // every wave takes the same barriers, whatever its TMV
  auto run = [&](auto tmv_c) {
    for (int c = 0; c < WC; ++c) issue_w(0, c);
    for (int c = 0; c < XI; ++c) issue_x(0, c);
    for (int s = 0; s < nk; ++s) {
      // step s's activations landed, and everything issued before them (its
      // weight stage); the next weight stage, issued after them at step s - 1
      // when s is odd, may stay in flight
      const bool w_after = (s & 1) && (s >> 1) + 1 < nu;
      wait_copies_barrier_n(w_after ? WC : 0);
      compute(s, tmv_c);
    }
  };
  if (nrows > 96)
    run(std::integral_constant<int, 4>{});
  else if (nrows > 64)
    run(std::integral_constant<int, 3>{});
  else if (nrows > 32)
    run(std::integral_constant<int, 2>{});
  else
    run(std::integral_constant<int, 1>{});

  // ---- epilogue: bf16, rotation Y^T_blk = R_j Z^T_blk on the matrix cores
  // (EPI_ROT*), store; SwiGLU pairs gate and up outputs through LDS.  The
  // last wait above took every copy, so the LDS is free after a barrier.
  const int nb = chan(32 * wave);  // first channel of this wave's 32
  const bool n_ok = nb >= 0;
  uint32_t swg[SWI ? TM : 1][8];
  bf16x8 ra[2];
  if constexpr (epi_rotates(EPI)) {
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
    f32x16 o;
    if constexpr (epi_rotates(EPI)) {
      const f32x16& z = acc[tm];
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
      o = acc[tm];
    }
    const int ml = 32 * tm + l32;
    const bool m_ok = n_ok && ml < nrows;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = pack_bf16x2(o[4 * q], o[4 * q + 1]);
      const uint32_t hi = pack_bf16x2(o[4 * q + 2], o[4 * q + 3]);
      if constexpr (SWI) {
        swg[tm][2 * q] = lo;
        swg[tm][2 * q + 1] = hi;
      }
      if (m_ok && (!SWI || p.out != nullptr)) {  // gate/up: the h store is optional
        const size_t off = (size_t)(pos0 + ml) * p.ldo + nb + 8 * q + 4 * g2;
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) = make_uint2(lo, hi);
      }
    }
  }

  if constexpr (SWI) {
    // up waves (4..7) hand their bf16 outputs to the gate waves (wave - 4)
    // holding the same (token, channel) slots, through the activation ring
    static_assert(4 * TM * 8 * 64 * 4 <= 2 * XB, "exchange buffer");
    uint32_t* xb = reinterpret_cast<uint32_t*>(xs);
    const int pid = wave & 3;
    lds_barrier_plain();
    if (wave >= 4) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int v = 0; v < 8; ++v) xb[((pid * TM + tm) * 8 + v) * 64 + lane] = swg[tm][v];
    }
    lds_barrier_plain();
    if (wave < 4 && nb >= 0) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int ml = 32 * tm + l32;
        if (ml >= nrows) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float av[4];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t gw = swg[tm][2 * q + h];
            const uint32_t uw = xb[((pid * TM + tm) * 8 + 2 * q + h) * 64 + lane];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
              const float gv = bf16_to_f32((uint16_t)(gw >> (16 * v)));
              const float uv = bf16_to_f32((uint16_t)(uw >> (16 * v)));
              av[2 * h + v] = gv / (1.0f + __expf(-gv)) * uv;
            }
          }
          *reinterpret_cast<uint2*>(p.act + (size_t)(pos0 + ml) * p.ldact + nb + 8 * q + 4 * g2) =
              make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
        }
      }
    }
  }
}

}  // namespace oft
