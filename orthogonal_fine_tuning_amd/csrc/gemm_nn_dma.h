// Backward-type dequant GEMM with asynchronous global -> LDS copies:
//   C^T[k][m] = sum_n W[n][k] B[m][n]
// The contraction runs over the weight's rows n (the weight as stored, no
// transposed copy); B rows are bf16, dense rows or gathered expert positions
// as in gemm_nn.h (kslots > 0: row perm[pos] / kslots); the epilogues are
// EPI_STORE and EPI_SWIGLU_BWD of gemm_nn.h (bf16 out).  Weights: INT4 codes
// with fp16 group scales, or bf16 (the dequantised reference).
//
// Workgroup: 8 waves, tile 256 output columns x 128 rows, contraction steps
// of 64 weight rows.  Wave (wk, wm) = (wave % 4, wave / 4) owns columns
// 64 wk + [0, 64) and rows 64 wm + [0, 64).
//
// Every HBM read of the main loop is a global_load_lds copy, counted by the
// kernel itself (vmcnt) as in gemm_nt_dma.h:
//   B tile   : 128 rows x 128 bytes, 16-byte chunk c of row r at c ^ swz_x(r);
//   INT4     : codes, 64 rows x 128 bytes in natural order, and each row's
//              fp16 group scales for the tile's columns as whole 4-byte
//              words (one word more than the scales fill, so that an odd
//              first scale index is covered);
//   bf16 W   : 64 rows x 512 bytes, chunk c of row n at c ^ 4 (n % 4).
// INT4 codes are dequantised once per workgroup, one step ahead of their
// use: thread (row n = t / 8, 32-column group q = t % 8) reads 16 code bytes
// and one scale and writes bf16(q s), 64 bytes, into a double-buffered tile
// with the bf16-W layout; its four 16-byte chunks go out in the order
// rotated by q / 2.  Both that layout (for the transpose loads below) and
// that order (for the writes) were measured free of LDS bank conflicts on
// gfx950; the plain order is four-way conflicted.
//
// Pipeline, one barrier per step s: B tiles three deep, issued two steps
// ahead; INT4 codes three deep, issued three steps ahead and dequantised one
// step ahead (bf16 W: three deep, two ahead).  The barrier of step s
// publishes the B tile of s, the bf16 tile of s (dequantised during step
// s - 1) and the codes of s + 1, and retires every read of step s - 1, whose
// buffers the copies and the dequant of step s then overwrite.
//
// Matrix-core operands (v_mfma_f32_32x32x16_bf16): A = W^T, rows = 32
// output columns k, contraction along n, read with the LDS transpose load
// ds_read_b64_tr_b16 (within each 16-lane group, lane i receives element
// i % 4 of the 8-byte pieces loaded by lanes 4e + i / 4: pointing lane r at
// row n0 + r / 4, column k0 + 4 (r % 4) gives lane i the values
// W[n0 .. n0 + 3][k0 + i]; two loads cover n0 .. n0 + 7); B = one 16-byte
// read of the B tile.  In MFMA kk (0..3) of a step, lane group g2 takes the
// contraction indices 32 g2 + 8 kk + p (p = 0..7) for both operands.
#pragma once

#include <type_traits>

#include "gemm_nn.h"
#include "gemm_nt_dma.h"

namespace oft {

namespace nnd {
constexpr int BKO = 256;                   // output columns per workgroup
constexpr int BNS = 64;                    // weight rows per step
constexpr int BM = 128;                    // rows (tokens / positions)
constexpr int NTHR = 512;
constexpr int NST = 3;                     // ring depth
constexpr int B_BYTES = BM * BNS * 2;      // B tile
constexpr int WROW = BKO * 2;              // bf16 weight row
constexpr int W_BYTES = BNS * WROW;        // bf16 weight tile
constexpr int C_BYTES = BNS * BKO / 2;     // INT4 codes
constexpr int S_WORDS = 5;                 // scale words per row at most (g = 32)
constexpr int CS_BYTES = C_BYTES + BNS * S_WORDS * 4;
// chunk (16 bytes) c of bf16 weight row n is stored at c ^ wsw(n)
__device__ __forceinline__ int wsw(int n) { return 4 * (n & 3); }
}  // namespace nnd

template <int WF, int EPI, bool GROUPED>
__global__ __launch_bounds__(nnd::NTHR, 1) void gemm_nn_dma_kernel(NnArgs p) {
  using namespace nnd;
  using ntd::copy16;
  using ntd::copy16v;
  using ntd::copy4;
  using ntd::lds_addr;
  using ntd::swz_x;
  static_assert((wf_4bit(WF) && !wf_tiled(WF)) || WF == WF_BF16, "row-major weights");
  static_assert(EPI == EPI_STORE || EPI == EPI_SWIGLU_BWD, "epilogue");
  constexpr bool W16 = WF == WF_BF16;
  constexpr int TM = BM / 64;  // 32-row tiles per wave
  // LDS: B ring, then the weight ring (bf16) or the code ring + two bf16 tiles
  constexpr int OFF_W = NST * B_BYTES;
  constexpr int OFF_D = OFF_W + NST * CS_BYTES;
  constexpr int LDS_BYTES = W16 ? OFF_W + NST * W_BYTES : OFF_D + 2 * W_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave & 3, wm = wave >> 2;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;
  const int ns = p.N / BNS;  // the host guarantees N % 64 == 0

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
  const int kbase = cx * BKO;
  const uint8_t* wc = p.wc + (size_t)e * p.wc_e;
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws) + (size_t)e * p.ws_e;

  // ---- B tile copies: rows 16 wave + 8 i + lane / 8 (past the end: row 0)
  const uint8_t* bbase = reinterpret_cast<const uint8_t*>(p.src) + (size_t)pos0 * p.lds * 2;
  uint32_t boff[2];
  const uint8_t* bptr[GROUPED ? 2 : 1];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wave + 8 * i + (lane >> 3);
    const int rr = r < nrows ? r : 0;
    const int chunk = 16 * ((lane & 7) ^ swz_x(r));
    boff[i] = (uint32_t)(rr * p.lds * 2 + chunk);
    if constexpr (GROUPED) {
      const long src = p.kslots > 0 ? (long)(p.perm[pos0 + rr] / p.kslots) : (long)(pos0 + rr);
      bptr[i] = reinterpret_cast<const uint8_t*>(p.src) + src * p.lds * 2 + chunk;
    }
  }
  const uint32_t b_lds = lds_addr(smem) + (uint32_t)(16 * wave * 128);

  // ---- weight copies
  const uint32_t w_lds = lds_addr(smem + OFF_W);
  uint32_t woff[4] = {0u, 0u, 0u, 0u};
  uint32_t soff = 0u;       // INT4: this lane's scale word (step 0)
  uint32_t s_dst = 0u;      // INT4: LDS word slot of this wave's scale copy
  int dpr = 0;              // INT4: scale words per row
  if constexpr (W16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 8 * wave + 2 * i + (lane >> 5);
      int c = (lane & 31) ^ wsw(n);
      if (kbase + 8 * c >= K) c = 0;  // past the last column: any valid piece
      woff[i] = (uint32_t)(n * K * 2 + (kbase + 8 * c) * 2);
    }
  } else {
    const int n = 8 * wave + (lane >> 3);
    int c = lane & 7;
    if (kbase + 32 * c >= K) c = 0;
    woff[0] = (uint32_t)(n * (K / 2) + kbase / 2 + 16 * c);
    const int kg = K / p.g;
    dpr = BKO / p.g / 2 + 1;
    const int d = (wave * 64 + lane) % (64 * dpr);
    const int rs = d / dpr, j = d % dpr;
    const int ng = min(BKO, K - kbase) / p.g;  // groups in this tile
    const int x = rs * kg + kbase / p.g;        // fp16 index of the row's first scale
    const int w0 = x >> 1, wl = (x + ng - 1) >> 1;
    soff = (uint32_t)(4 * (w0 + min(j, wl - w0)));
    s_dst = (uint32_t)(4 * ((wave * 64) % (64 * dpr)));
  }

  // B copies of this wave that hold a row of the tile (the rest would only
  // copy rows past its end, whose products are never stored: skipped)
  const int vb = (16 * wave < nrows ? 1 : 0) + (16 * wave + 8 < nrows ? 1 : 0);
  auto issue_b = [&](int s) {
    const uint32_t dst = b_lds + (uint32_t)((s % NST) * B_BYTES);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= vb) break;
      if constexpr (GROUPED)
        copy16v(dst + i * 1024, bptr[i] + (size_t)s * BNS * 2);
      else
        copy16(dst + i * 1024, bbase + (size_t)s * BNS * 2, boff[i]);
    }
  };
  auto issue_w = [&](int s) {
    if constexpr (W16) {
      const uint32_t dst = w_lds + (uint32_t)((s % NST) * W_BYTES + 8 * wave * WROW);
      const uint8_t* src = wc + (size_t)s * BNS * K * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) copy16(dst + i * 1024, src, woff[i]);
    } else {
      const uint32_t dst = w_lds + (uint32_t)((s % NST) * CS_BYTES);
      copy16(dst + wave * 1024, wc + (size_t)s * BNS * (K / 2), woff[0]);
      copy4(dst + C_BYTES + s_dst, reinterpret_cast<const uint8_t*>(ws_h) + (size_t)s * BNS * (K / p.g) * 2, soff);
    }
  };

  // ---- INT4 dequant of step s into bf16 tile s % 2
  const int dq_r = tid >> 3, dq_q = tid & 7;
  const int dq_rot = (dq_q >> 1) & 3;
  int dq_sidx = 0;  // fp16 index of this thread's scale within its row's words
  if constexpr (!W16) dq_sidx = ((dq_r * (K / p.g) + kbase / p.g) & 1) + (32 * dq_q) / p.g;
  auto dequant = [&](int s) {
    if constexpr (!W16) {
      const uint8_t* C = smem + OFF_W + (s % NST) * CS_BYTES;
      const uint4 cw = *reinterpret_cast<const uint4*>(C + dq_r * 128 + 16 * dq_q);
      const uint16_t sb = *reinterpret_cast<const uint16_t*>(C + C_BYTES + dq_r * dpr * 4 + 2 * dq_sidx);
      const auto sc = W4<WF>::scale(sb);
      // rotate the four code words by dq_rot: output i is chunk (i + rot) % 4
      uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
      uint32_t v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (dq_rot & 1) ? w[(i + 1) & 3] : w[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (dq_rot & 2) ? v[(i + 2) & 3] : v[i];
      uint8_t* D = smem + OFF_D + (s & 1) * W_BYTES + dq_r * WROW;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 4 * dq_q + ((i + dq_rot) & 3);
        *reinterpret_cast<uint4*>(D + 16 * (c ^ wsw(dq_r))) = W4<WF>::dq(w[i], sc);
      }
    }
  };

  // ---- operand addresses
  const int G = lane >> 4, li = lane & 15;
  uint32_t ard[2][4];  // [tk][kk] byte offset of the A transpose load (rows n0 .. n0 + 3)
#pragma unroll
  for (int tk = 0; tk < 2; ++tk)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int n = 32 * (G >> 1) + 8 * kk + (li >> 2);
      const int k = 64 * wk + 32 * tk + 16 * (G & 1) + 4 * (li & 3);
      ard[tk][kk] = (uint32_t)(n * WROW + 16 * ((k >> 3) ^ wsw(n)) + 2 * (k & 7));
    }
  const int xsw = swz_x(l32);
  uint32_t brd[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) brd[tm] = (uint32_t)((64 * wm + 32 * tm + l32) * 128);

  f32x16 acc[2][TM];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // TMV (a std::integral_constant): this wave's 32-row tiles that hold rows
  auto compute = [&](int s, auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    if constexpr (TMV > 0) {
      const uint8_t* Bt = smem + (s % NST) * B_BYTES;
      const uint16_t* At = reinterpret_cast<const uint16_t*>(
          W16 ? smem + OFF_W + (s % NST) * W_BYTES : smem + OFF_D + (s & 1) * W_BYTES);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 a[2], b[TMV];
#pragma unroll
        for (int tk = 0; tk < 2; ++tk) {
          const uint16_t* q0 = At + ard[tk][kk] / 2;
          const uint2 lo = nn::ds_read_tr16(q0);
          const uint2 hi = nn::ds_read_tr16(q0 + 4 * WROW / 2);
          a[tk] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
#pragma unroll
        for (int tm = 0; tm < TMV; ++tm)
          b[tm] = *reinterpret_cast<const bf16x8*>(Bt + brd[tm] + 16 * ((4 * g2 + kk) ^ xsw));
#pragma unroll
        for (int tk = 0; tk < 2; ++tk)
#pragma unroll
          for (int tm = 0; tm < TMV; ++tm) acc[tk][tm] = mfma32(a[tk], b[tm], acc[tk][tm]);
      }
    }
  };

  // copies issued per wave and step: B vb (0 .. 2), weights 4 (bf16) or 2
  // (codes + scales)
  const int VB = vb;
  constexpr int VW = W16 ? 4 : 2;
  auto run = [&](auto tmv_c) {
    if constexpr (W16) {
      issue_w(0);
      issue_b(0);
      if (ns > 1) {
        issue_w(1);
        issue_b(1);
      }
      for (int s = 0; s < ns; ++s) {
        ntd::wait_copies_barrier_n(s + 1 < ns ? VB + VW : 0);
        if (s + 2 < ns) {
          issue_w(s + 2);
          issue_b(s + 2);
        }
        compute(s, tmv_c);
      }
    } else {
      issue_w(0);
      if (ns > 1) issue_w(1);
      issue_b(0);
      // step s = -1 only dequantises the codes of step 0
      for (int s = -1; s < ns; ++s) {
        // copies of the previous step (codes of s + 2, B tile of s + 1) may
        // stay in flight
        ntd::wait_copies_barrier_n((s + 2 < ns ? VW : 0) + (s + 1 < ns ? VB : 0));
        if (s + 3 < ns) issue_w(s + 3);
        if (s + 2 < ns) issue_b(s + 2);
        if (s + 1 < ns) dequant(s + 1);
        if (s >= 0) compute(s, tmv_c);
      }
    }
  };
  const int rows_w = nrows - 64 * wm;  // rows of this wave's 64 (uniform)
  if (rows_w > 32)
    run(std::integral_constant<int, 2>{});
  else if (rows_w > 0)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});

  // ------------------------------------------------------------ epilogue
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int tk = 0; tk < 2; ++tk) {
      const int kb = kbase + 64 * wk + 32 * tk;
      if (kb >= K) continue;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int ml = 64 * wm + 32 * tm + l32;
        if (ml >= nrows) continue;
        const f32x16& o = acc[tk][tm];
        uint16_t* orow = static_cast<uint16_t*>(p.out) + (size_t)(pos0 + ml) * p.ldo + kb;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(orow + 8 * q + 4 * g2) =
              make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
      }
    }
  } else {
    // SwiGLU backward (as gemm_nn.h); out = dH [P, 2I] with ldo, K = I
    float dwp[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      dwp[tm] = 0.0f;
      const int ml = 64 * wm + 32 * tm + l32;
      const bool m_ok = ml < nrows;
      const long pos = (long)(pos0 + ml);
      const float wgt = m_ok ? p.topk_w[p.perm[pos]] : 0.0f;
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        const int kb = kbase + 64 * wk + 32 * tk;
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
    // per-position partial over this 256-column tile: lanes g2 = 0/1, then
    // the four wk waves in fixed order through LDS (the ring is free once
    // every wave has passed the barrier)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) dwp[tm] += __shfl_xor(dwp[tm], 32);
    float* red = reinterpret_cast<float*>(smem);
    ntd::lds_barrier_plain();
    if (g2 == 0) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) red[wk * BM + 64 * wm + 32 * tm + l32] = dwp[tm];
    }
    ntd::lds_barrier_plain();
    if (wk == 0 && g2 == 0) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int ml = 64 * wm + 32 * tm + l32;
        if (ml < nrows)
          p.dw_part[(size_t)cx * p.P + pos0 + ml] =
              ((red[ml] + red[BM + ml]) + red[2 * BM + ml]) + red[3 * BM + ml];
      }
    }
  }
}

}  // namespace oft
