// Dense dequant GEMM with asynchronous global -> LDS copies (bf16 x):
//   C^T[n][m] = sum_k W[n][k] x[m][k]
// with W as FP8 or 4-bit codes (the forward, EPI_ROT: the rotation epilogue
// of gemm_nt.h) or as bf16 (EPI_PLAIN: plain store; the backward's dX runs
// here with W = the transposed, dequantised weight and x = the rotated
// upstream gradient).
//
// Grouped (MoE experts): tile y is entry y of a device work list (expert e,
// row0) as in gemm_nt.h; its rows are expert-sorted positions, activation
// rows are gathered (row perm[pos] / kslots) by per-lane 64-bit copy
// addresses, and the weight, scale and rotation pointers advance by expert.
// EPI_ROT_SWIGLU: the 256-channel tile is 128 gate channels [c, c + 128) and
// the matching 128 up channels [I + c, I + c + 128); both are rotated and
// stored, then act = silu(gate) * up, the up waves handing their bf16
// outputs to the gate waves through LDS.  EPI_BASE_SWIGLU: the same without
// the rotation (the frozen base alone), h stored only when out is set.
//
// Workgroup: 8 waves, tile 256 channels x BM tokens (BM = 128 or 192), K
// steps of 64.  FP8 and bf16 weights: wave (wn, wm) = (wave % 4, wave / 4)
// owns channels 64 wn + [0, 64) and tokens wm BM / 2 + [0, BM / 2).  INT4
// weights on 128-token tiles: wave wn owns channels 32 wn + [0, 32) and every
// token, so each code row is dequantised by one wave only (with the 4 x 2
// layout both token halves dequantised it, and on 128-token tiles the
// dequant, not the matrix cores, set the pace).
//
// Everything the main loop reads from HBM travels by global_load_lds (16 or
// 4 bytes per lane; lane l of an instruction writes LDS bytes [s l, s l + s)
// after the wave-uniform base in M0), through a ring of three LDS stages:
//   activations : BM rows x 128 bytes (one full cache line per row);
//   weights     : 256 rows x 64 bytes (FP8) or x 32 bytes plus one 4-byte
//                 word per row holding its fp16 group scale(s) (INT4), or
//                 x 128 bytes (bf16, laid out like the activations).
// Each wave copies an eighth of both.  The copies for step s + 2 are issued
// during step s, right after its first group of matrix-core instructions,
// so each has two steps of matrix-core work to land; no registers hold data
// in flight.  The kernel counts its
// copies itself (vmcnt): they are assembly, so the compiler neither waits
// for them before unrelated LDS reads nor miscounts its own loads around
// them, and the loop issues no other global loads.  One barrier per step:
// it publishes step s and retires the reads of step s - 1, whose stage the
// copies of step s + 2 then overwrite.
//
// Weights are dequantised by the waves that multiply them, from the LDS
// codes straight into matrix-core operands (FP8: exact conversion, its
// per-channel scale applied in the fp32 epilogue; INT4: bf16(q s) with the
// group scale, the same values as the dequant hook).
//
// Contraction order: in MFMA kk (0..3) of a step, lane group g2 takes the
// in-features 32 g2 + 8 kk + p (p = 0..7) for both operands, so a lane's
// weight codes for the whole step are contiguous (32 FP8 or 16 INT4 bytes)
// and each activation operand is one 16-byte read.
//
// LDS layouts: 16-byte chunk c of a row r sits at chunk c ^ h(r), with
// h = (r ^ ((r >> 3) & 1)) & 7 for activation rows (8 chunks; bf16 weight
// rows too), (r >> 2) & 3 for FP8 code rows (4 chunks) and
// ((r >> 2) ^ (r >> 3)) & 1 for INT4 code rows (2).  Each was measured free
// of bank conflicts for the operand reads on gfx950 (bank-conflict counter
// and read rate of a probe kernel, against contiguous reads); the earlier
// FP8 choice ((r >> 1) ^ (r >> 3)) & 3 ran at half rate.
#pragma once

#include <type_traits>

#include "gemm_nt.h"

namespace oft {

namespace ntd {
constexpr int BN = 256;  // channels per workgroup
constexpr int BK = 64;   // in-features per step
constexpr int NST = 3;   // ring depth
constexpr int NTHR = 512;
template <int BM> constexpr int X_BYTES = BM * BK * 2;
template <int WF> constexpr int W_BYTES = WF == WF_BF16 ? BN * BK * 2 : WF == WF_FP8 ? BN * BK : BN * BK / 2 + BN * 4;
__device__ __forceinline__ int swz_x(int r) { return (r ^ ((r >> 3) & 1)) & 7; }
__device__ __forceinline__ int swz_w8(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_w4(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

// 16 (or 4) bytes per lane from base + voff to LDS byte address lds + 16 l (4 l)
__device__ __forceinline__ void copy16(uint32_t lds, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void copy16v(uint32_t lds, const void* addr) {  // per-lane 64-bit address
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(addr) : "memory", "m0");
}
__device__ __forceinline__ void copy4(uint32_t lds, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}
// 2 bytes per lane into the LDS dword slot of the lane (zero-extended)
__device__ __forceinline__ void copy2(uint32_t lds, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}
// wait until at most N copies of this wave are in flight, then a workgroup
// barrier that also retires this wave's LDS reads
template <int N>
__device__ __forceinline__ void wait_copies_barrier() {
  static_assert(N == 0 || N == 4 || N == 5 || N == 6 || N == 8, "copies per step");
  if constexpr (N == 0)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 5)
    asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4)
    asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 6)
    asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// runtime count 0 .. 16 (a larger count waits for all)
__device__ __forceinline__ void wait_copies_barrier_n(int n) {
#define OFT_WCB(N) \
  case N: asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  switch (n) {
    OFT_WCB(16) OFT_WCB(15) OFT_WCB(14) OFT_WCB(13) OFT_WCB(12) OFT_WCB(11) OFT_WCB(10) OFT_WCB(9)
    OFT_WCB(8) OFT_WCB(7) OFT_WCB(6) OFT_WCB(5) OFT_WCB(4) OFT_WCB(3) OFT_WCB(2) OFT_WCB(1)
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
#undef OFT_WCB
}
// workgroup barrier after this wave's LDS accesses have completed
__device__ __forceinline__ void lds_barrier_plain() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
}  // namespace ntd

template <int WF, int B, int BM, int EPI, bool OUTF32, bool GROUPED = false, int KB = 64>
__global__ __launch_bounds__(ntd::NTHR, (WF != WF_BF16 && BM == 128 && KB == 64) ? 2 : 1) void gemm_nt_dma_kernel(
    NtArgs p) {
  using namespace ntd;
  static_assert(KB == 64 || (KB == 128 && WF == WF_FP8 && BM <= 192 && !GROUPED), "128-wide K steps: FP8, <= 192 tokens");
  static_assert(BM == 128 || BM == 192, "tile");
  static_assert(WF != WF_BF16 || BM == 128, "bf16 weights: three stages fit with 128-token tiles only");
  static_assert(!wf_tiled(WF), "row-major weights only");
  static_assert(EPI == EPI_ROT || EPI == EPI_PLAIN || epi_swiglu(EPI) || EPI == EPI_BASE, "epilogue");
  static_assert(!epi_swiglu(EPI) || BM == 128, "exchange buffer sized for 128-token tiles");
  constexpr bool FP8 = WF == WF_FP8;
  constexpr bool W16 = WF == WF_BF16;
  constexpr bool SWI = epi_swiglu(EPI);
  // wave layout: INT4 weights on 128-token tiles, 8 waves x 32 channels over
  // every token of the tile (each code row is dequantised by one wave only);
  // otherwise 4 x 2 waves of 64 channels x BM / 2 tokens
  constexpr bool W8 = wf_4bit(WF) && BM == 128;
  constexpr int TN = W8 ? 1 : 2;              // 32-channel tiles per wave
  constexpr int TM = W8 ? BM / 32 : BM / 64;  // 32-token tiles per wave
  constexpr int NWN = W8 ? 8 : 4;             // waves along the channels
  // K steps of KB in-features: 64 (three stages, copies two steps ahead) or
  // 128 (FP8 on 192-token tiles: two stages of 80 KB, copies one step ahead,
  // half the barriers).  128-token tiles run two workgroups per CU, so that
  // one's barrier waits are covered by the other's matrix work: INT4 fits
  // with three stages (77 KB), FP8 with two stages of 64-wide steps (64 KB;
  // measured faster than one workgroup with 128-wide steps)
  constexpr bool TWO = WF == WF_FP8 && BM == 128 && KB == 64;
  constexpr int NSTK = (KB == 128 || TWO) ? 2 : NST;
  constexpr int LA = NSTK - 1;               // copy lookahead in steps
  constexpr int XROW = KB * 2;               // activation row bytes per step
  constexpr int XB = BM * XROW;
  constexpr int WB = KB == 128 ? BN * KB : W_BYTES<WF>;
  constexpr int XI = XB / 8 / 1024;          // activation copies per wave and step
  constexpr int WI = W16 ? 4 : FP8 ? KB / 32 : 2;  // weight copies per wave and step
  constexpr int V = XI + WI;                 // copies per wave and step
  constexpr int NKK = KB / 16;               // MFMA groups per step
  static_assert(NSTK * (XB + WB) <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) uint8_t xs[NSTK * XB];
  __shared__ __attribute__((aligned(16))) uint8_t wsm[NSTK * WB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = W8 ? wave : (wave & 3), wm = W8 ? 0 : (wave >> 2);
  const int cw0 = W8 ? 32 * wn : 64 * wn;  // this wave's first weight row of the tile
  const int rw0 = W8 ? 0 : wm * (BM / 2);  // and first token row
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;

  // ---- tile: rows (tokens / expert positions) and weight rows (channels)
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
  // channel of local weight row rw (0..255), or -1 past the layer's channels
  const int cbase = SWI ? cx * (BN / 2) : cx * BN;
  auto chan = [&](int rw) -> int {
    if constexpr (SWI) {
      const int c = cbase + (rw & (BN / 2 - 1));
      return c < p.half_n ? (rw < BN / 2 ? c : p.half_n + c) : -1;
    } else {
      return cbase + rw < p.N ? cbase + rw : -1;
    }
  };
  // copy source row: invalid rows copy the workgroup's first row (never stored)
  auto crow = [&](int rw) { const int c = chan(rw); return c >= 0 ? c - cbase : 0; };
  const int nk = K / KB;
  const int kg = wf_4bit(WF) ? K / p.g : 1;  // 4-bit scales per row
  const int gs = p.g == 32 ? 1 : p.g == 64 ? 0 : -1;  // INT4: log2(64 / g)

  // ---- copy sources: activations (dense: per-lane 32-bit offsets from the
  // tile's first row; grouped: per-lane 64-bit addresses of gathered rows)
  const uint8_t* xbase = static_cast<const uint8_t*>(p.a) + (size_t)pos0 * p.lda * 2;
  uint32_t xoff[XI];
  const uint8_t* xptr[GROUPED ? XI : 1];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    // one copy = 1 KB: 8 rows of 128 bytes (KB = 64) or 4 rows of 256 bytes
    const int r = KB == 128 ? (BM / 8) * wave + 4 * i + (lane >> 4) : (BM / 8) * wave + 8 * i + (lane >> 3);
    const int rr = r < nrows ? r : 0;  // rows past the end copy row 0; never stored
    const int chunk = KB == 128 ? 16 * ((lane & 15) ^ (r & 15)) : 16 * ((lane & 7) ^ swz_x(r));
    xoff[i] = (uint32_t)(rr * p.lda * 2 + chunk);
    if constexpr (GROUPED) {
      const long src = p.kslots > 0 ? (long)(p.perm[pos0 + rr] / p.kslots) : (long)(pos0 + rr);
      xptr[i] = static_cast<const uint8_t*>(p.a) + src * p.lda * 2 + chunk;
    }
  }
  const uint32_t x_lds = lds_addr(xs) + (uint32_t)((BM / 8) * wave * XROW);
  // activation copies of this wave that hold a row of the tile (a prefix of
  // the XI; the rest would only copy rows past the tile's end, whose
  // products are never stored: skipped, and the wave's copy count per step
  // drops accordingly)
  int xc = 0;
#pragma unroll
  for (int i = 0; i < XI; ++i) xc += (BM / 8) * wave + (KB == 128 ? 4 : 8) * i < nrows ? 1 : 0;
  const int vw = xc + WI;  // copies per step of this wave

  // weights: per-lane 32-bit offsets from the row of channel cbase
  const uint8_t* wbase = wc + (W16 ? (size_t)cbase * K * 2 : FP8 ? (size_t)cbase * K : (size_t)cbase * (K / 2));
  uint32_t woff[4] = {0u, 0u, 0u, 0u};
  uint32_t sbase = 0;  // INT4: index of the copy row's first scale
  if constexpr (W16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rw = 32 * wave + 8 * i + (lane >> 3);
      woff[i] = (uint32_t)(crow(rw) * K * 2 + 16 * ((lane & 7) ^ swz_x(rw)));
    }
  } else if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      if constexpr (KB == 128) {  // 128-byte rows, chunk c at c ^ ((r >> 1) & 7)
        const int rw = 32 * wave + 8 * i + (lane >> 3);
        woff[i] = (uint32_t)(crow(rw) * K + 16 * ((lane & 7) ^ ((rw >> 1) & 7)));
      } else {
        const int rw = 32 * wave + 16 * i + (lane >> 2);
        woff[i] = (uint32_t)(crow(rw) * K + 16 * ((lane & 3) ^ swz_w8(rw)));
      }
    }
  } else {
    const int rw = 32 * wave + (lane >> 1);
    woff[0] = (uint32_t)(crow(rw) * (K / 2) + 16 * ((lane & 1) ^ swz_w4(rw)));
    sbase = (uint32_t)((cbase + crow(32 * wave + l32)) * kg);
  }
  const uint32_t w_lds = lds_addr(wsm) + (uint32_t)(32 * wave * (W16 ? 128 : FP8 ? KB : 32));
  const uint32_t s_lds = lds_addr(wsm) + (uint32_t)(BN * BK / 2 + 32 * wave * 4);
  // first scale of step s: (64 s) / g
  auto sstep = [&](int s) { return gs >= 0 ? s << gs : s >> 1; };

  // copy c (0 .. V - 1) of step s: activations first, then weights
  auto copy_one = [&](int s, int c) {
    const int st = s % NSTK;
    if (c < XI) {
      if (c >= xc) return;
      if constexpr (GROUPED)
        copy16v(x_lds + st * XB + c * 1024, xptr[c] + (size_t)s * XROW);
      else
        copy16(x_lds + st * XB + c * 1024, xbase + (size_t)s * XROW, xoff[c]);
      return;
    }
    const int i = c - XI;
    if constexpr (W16) {
      copy16(w_lds + st * WB + i * 1024, wbase + (size_t)s * BK * 2, woff[i]);
    } else if constexpr (FP8) {
      copy16(w_lds + st * WB + i * 1024, wbase + (size_t)s * KB, woff[i]);
    } else if (i == 0) {
      copy16(w_lds + st * WB, wbase + (size_t)s * (BK / 2), woff[0]);
    } else {
      // lanes 0..31: the 4-byte word holding the step's scale(s) of row 32 wave + lane
      if (lane < 32) copy4(s_lds + st * WB, ws_h, ((sbase + (uint32_t)sstep(s)) * 2u) & ~3u);
    }
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int c = 0; c < V; ++c) copy_one(s, c);
  };

  // ---- operand reads
  uint32_t xrd[TM];  // activation row r = rw0 + 32 tm + l32
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) xrd[tm] = (uint32_t)((rw0 + 32 * tm + l32) * XROW);
  // the swizzle depends on bits 0..3 of the row only: the same for every tm, wm
  const int xsw = KB == 128 ? (l32 & 15) : swz_x(l32);
  const int xg = KB == 128 ? 8 * g2 : 4 * g2;  // first chunk of this lane group's in-features
  uint32_t wrd[2][4];
  uint32_t srd[2] = {0u, 0u};  // INT4: scale index of the operand row at k = 0
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int rw = cw0 + 32 * tn + l32;
    if constexpr (W16) {
      wrd[tn][0] = (uint32_t)(rw * 128);
      wrd[tn][1] = 0u;
    } else if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < KB / 32; ++j)
        wrd[tn][j] = KB == 128 ? (uint32_t)(rw * 128 + 16 * ((4 * g2 + j) ^ ((rw >> 1) & 7)))
                               : (uint32_t)(rw * 64 + 16 * ((2 * g2 + j) ^ swz_w8(rw)));
    } else {
      wrd[tn][0] = (uint32_t)(rw * 32 + 16 * (g2 ^ swz_w4(rw)));
      wrd[tn][1] = 0u;
      srd[tn] = (uint32_t)((cbase + crow(rw)) * kg);
    }
  }

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // iss: issue the copies of step s + 2 once the first matrix-core group of
  // step s is queued, so that a stalled copy issue overlaps matrix work.
  // TMV (a std::integral_constant): this wave's 32-token tiles that hold
  // rows; the others are skipped (grouped tiles past an expert's last row).
  auto compute = [&](int s, bool iss, auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    const int st = s % NSTK;
    const uint8_t* X = xs + st * XB;
    const uint8_t* W = wsm + st * WB;
    if constexpr (TMV == 0) {
      if (iss) issue(s + LA);
      return;
    }
    uint32_t cw[TN][KB / 4];  // this lane's codes for the step (INT4: words 0..3)
    typename W4<WF>::S sc[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if constexpr (W16) {
        // bf16 weight rows are read per MFMA below, like the activations
      } else if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < KB / 32; ++j) {
          const uint4 c = *reinterpret_cast<const uint4*>(W + wrd[tn][j]);
          cw[tn][4 * j] = c.x; cw[tn][4 * j + 1] = c.y; cw[tn][4 * j + 2] = c.z; cw[tn][4 * j + 3] = c.w;
        }
      } else {
        const uint4 c0 = *reinterpret_cast<const uint4*>(W + wrd[tn][0]);
        cw[tn][0] = c0.x; cw[tn][1] = c0.y; cw[tn][2] = c0.z; cw[tn][3] = c0.w;
        const int rw = cw0 + 32 * tn + l32;
        const uint32_t word = *reinterpret_cast<const uint32_t*>(W + BN * BK / 2 + rw * 4);
        // this lane's in-features 64 s + 32 g2 .. + 31 lie in group (64 s + 32 g2) / g
        const uint32_t idx = srd[tn] + (uint32_t)(gs == 1 ? 2 * s + g2 : gs == 0 ? s : s >> 1);
        sc[tn] = W4<WF>::scale((uint16_t)(word >> (16 * (idx & 1))));
      }
    }
    // operands of MFMA group kk: weights (dequantised or read) and tokens
    auto make_a = [&](int kk, bf16x8* a) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if constexpr (W16) {
          a[tn] = *reinterpret_cast<const bf16x8*>(W + wrd[tn][0] + 16 * ((xg + kk) ^ xsw));
        } else if constexpr (FP8) {
          const uint2 lo = dq_fp8x4(cw[tn][2 * kk]), hi = dq_fp8x4(cw[tn][2 * kk + 1]);
          a[tn] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
          a[tn] = as_bf16x8(W4<WF>::dq(cw[tn][kk], sc[tn]));
        }
      }
    };
    auto load_b = [&](int kk, bf16x8* b) {
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm)
        b[tm] = *reinterpret_cast<const bf16x8*>(X + xrd[tm] + 16 * ((xg + kk) ^ xsw));
    };
    // one group ahead: the token reads and the dequant of group kk + 1 are
    // issued around the matrix instructions of group kk
    bf16x8 aq[2][TN], bq[2][TMV];
    load_b(0, bq[0]);
    make_a(0, aq[0]);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < NKK) load_b(kk + 1, bq[c ^ 1]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TMV; ++tm) acc[tn][tm] = mfma32(aq[c][tn], bq[c][tm], acc[tn][tm]);
      // the copies of step s + LA: bf16 weights and INT4 on 128-token tiles
      // spread them over the step's groups, the others issue them after the
      // first group (each measured faster that way)
      if (iss) {
        constexpr bool SPREAD = W16 || W8;
#pragma unroll
        for (int cc = 0; cc < V; ++cc)
          if (SPREAD ? (cc * NKK / V == kk) : kk == 0) copy_one(s + LA, cc);
      }
      if (kk + 1 < NKK) make_a(kk + 1, aq[c ^ 1]);
    }
  };

  // every wave takes the same barriers, whatever its TMV
  auto run = [&](auto tmv_c) {
    issue(0);
    if (LA > 1 && nk > 1) issue(1);
    for (int s = 0; s < nk; ++s) {
      // copies of steps s + 1 .. s + LA - 1 may stay in flight
      if constexpr (LA > 1) {
        wait_copies_barrier_n(s + 1 < nk ? vw : 0);
      } else {
        wait_copies_barrier<0>();
      }
      compute(s, s + LA < nk, tmv_c);
    }
  };
  if constexpr (GROUPED) {
    static_assert(BM == 128, "grouped tiles: 128 rows");
    const int rows_w = nrows - rw0;  // rows of this wave's tokens (uniform)
    if constexpr (TM == 4) {
      if (rows_w > 96)
        run(std::integral_constant<int, 4>{});
      else if (rows_w > 64)
        run(std::integral_constant<int, 3>{});
      else if (rows_w > 32)
        run(std::integral_constant<int, 2>{});
      else
        run(std::integral_constant<int, 1>{});
    } else {
      if (rows_w > 32)
        run(std::integral_constant<int, 2>{});
      else if (rows_w > 0)
        run(std::integral_constant<int, 1>{});
      else
        run(std::integral_constant<int, 0>{});
    }
  } else {
    run(std::integral_constant<int, TM>{});
  }

  // ------------------------------------------------------------ epilogue
  // EPI_ROT / EPI_ROT_SWIGLU: FP8 channel scale, bf16, Y^T_blk = R_j Z^T_blk
  // on the matrix cores (accumulator registers reused as the B operand),
  // store.  EPI_PLAIN: store the accumulators (bf16 or fp32).  EPI_BASE:
  // FP8 channel scale, store (no rotation).
  const float* ws_f = static_cast<const float*>(p.ws);
  uint32_t swg[SWI ? TN : 1][SWI ? TM : 1][8];  // EPI_ROT_SWIGLU: this lane's bf16 outputs
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int nb = chan(cw0 + 32 * tn);  // first channel of this 32-channel group
    const bool n_ok = nb >= 0;
    float fs[16];
    if constexpr (EPI != EPI_PLAIN && FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (n_ok) v = *reinterpret_cast<const float4*>(ws_f + nb + 8 * q + 4 * g2);
        fs[4 * q] = v.x;
        fs[4 * q + 1] = v.y;
        fs[4 * q + 2] = v.z;
        fs[4 * q + 3] = v.w;
      }
    }
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
        f32x16 z = acc[tn][tm];
        if constexpr (FP8) {
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] *= fs[r];
        }
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
        o = acc[tn][tm];
        if constexpr (EPI == EPI_BASE && FP8) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[r] *= fs[r];
        }
      }
      const int ml = rw0 + 32 * tm + l32;
      const bool m_ok = n_ok && ml < nrows;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = pack_bf16x2(o[4 * q], o[4 * q + 1]);
        const uint32_t hi = pack_bf16x2(o[4 * q + 2], o[4 * q + 3]);
        if constexpr (SWI) {
          swg[tn][tm][2 * q] = lo;
          swg[tn][tm][2 * q + 1] = hi;
        }
        if (m_ok && (!SWI || p.out != nullptr)) {  // gate/up: the h store is optional
          const size_t off = (size_t)(pos0 + ml) * p.ldo + nb + 8 * q + 4 * g2;
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

  if constexpr (SWI) {
    // up waves (the upper half of wn) hand their bf16 outputs to the gate
    // waves (wn - NWN / 2) holding the same (token, channel) slots; the ring
    // is free once every wave has passed the barrier
    static_assert(4 * TN * TM * 8 * 64 * 4 <= NSTK * XB, "exchange buffer");
    uint32_t* xb = reinterpret_cast<uint32_t*>(xs);
    const int pid = W8 ? (wn % (NWN / 2)) : (wn % (NWN / 2)) * 2 + wm;  // pair slot 0..3
    lds_barrier_plain();
    if (wn >= NWN / 2) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int v = 0; v < 8; ++v) xb[(((pid * TN + tn) * TM + tm) * 8 + v) * 64 + lane] = swg[tn][tm][v];
    }
    lds_barrier_plain();
    if (wn < NWN / 2) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int cb = chan(cw0 + 32 * tn);  // gate channel = act column
        if (cb < 0) continue;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int ml = rw0 + 32 * tm + l32;
          if (ml >= nrows) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float av[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t gw = swg[tn][tm][2 * q + h];
              const uint32_t uw = xb[(((pid * TN + tn) * TM + tm) * 8 + 2 * q + h) * 64 + lane];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float gv = bf16_to_f32((uint16_t)(gw >> (16 * u)));
                const float uv = bf16_to_f32((uint16_t)(uw >> (16 * u)));
                av[2 * h + u] = gv / (1.0f + __expf(-gv)) * uv;
              }
            }
            *reinterpret_cast<uint2*>(p.act + (size_t)(pos0 + ml) * p.ldact + cb + 8 * q + 4 * g2) =
                make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
          }
        }
      }
    }
  }
}

// Decode kernels' finish: the kh = 1 waves hand their partial sums to the
// kh = 0 waves through LDS (fixed order), which then run the epilogue: FP8
// channel scale, bf16, rotation (EPI_ROT*), store; EPI_ROT_SWIGLU passes the
// up outputs to the gate waves through LDS.  smem: SMEM bytes, free once
// every wave has passed the first barrier.  nb: first channel of the wave's
// 32 (-1 past the layer).
template <bool FP8, int B, int EPI, int TM, int SMEM, int KP = 2>
__device__ __forceinline__ void dec_finish(const NtArgs& p, f32x16 (&acc)[TM], uint8_t* smem, int wn, int kh,
                                           int lane, int nb, int nrows, int pos0, const uint16_t* rops) {
  using namespace ntd;
  constexpr bool SWI = epi_swiglu(EPI);
  static_assert(KP == 2 || (KP == 4 && !SWI), "k parts");
  static_assert((KP - 1) * 4 * TM * 16 * 64 * 4 <= SMEM, "partial-sum area");
  const int l32 = lane & 31, g2 = lane >> 5;
  // kh: this wave's part of the in-features of a step (0 .. KP - 1); parts
  // 1 .. KP - 1 hand their sums to part 0, which adds them in part order
  lds_barrier_plain();
  float* red = reinterpret_cast<float*>(smem);
  if (kh > 0) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((((kh - 1) * 4 + wn) * TM + tm) * 16 + r) * 64 + lane] = acc[tm][r];
  }
  lds_barrier_plain();
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < KP - 1; ++j)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tm][r] += red[(((j * 4 + wn) * TM + tm) * 16 + r) * 64 + lane];
  }

  // epilogue (kh = 0 waves): FP8 channel scale, bf16, rotation (EPI_ROT*), store
  const float* ws_f = static_cast<const float*>(p.ws);
  uint32_t swg[SWI ? TM : 1][8];
  if (kh == 0 && nb >= 0) {
    float fs[16];
    if constexpr (EPI != EPI_PLAIN && FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(ws_f + nb + 8 * q + 4 * g2);
        fs[4 * q] = v.x;
        fs[4 * q + 1] = v.y;
        fs[4 * q + 2] = v.z;
        fs[4 * q + 3] = v.w;
      }
    }
    bf16x8 ra[2];
    if constexpr (epi_rotates(EPI)) {
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
    for (int tm = 0; tm < TM; ++tm) {
      f32x16 o;
      if constexpr (epi_rotates(EPI)) {
        f32x16 z = acc[tm];
        if constexpr (FP8) {
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] *= fs[r];
        }
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
        if constexpr (EPI == EPI_BASE && FP8) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[r] *= fs[r];
        }
      }
      const int ml = 32 * tm + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = pack_bf16x2(o[4 * q], o[4 * q + 1]);
        const uint32_t hi = pack_bf16x2(o[4 * q + 2], o[4 * q + 3]);
        if constexpr (SWI) {
          swg[tm][2 * q] = lo;
          swg[tm][2 * q + 1] = hi;
        }
        if (ml < nrows && (!SWI || p.out != nullptr)) {  // gate/up: the h store is optional
          const size_t off = (size_t)(pos0 + ml) * p.ldo + nb + 8 * q + 4 * g2;
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) = make_uint2(lo, hi);
        }
      }
    }
  }
  if constexpr (SWI) {
    // up waves (wn = 2, 3) hand their bf16 outputs to the gate waves (wn =
    // 0, 1), in LDS past the partial-sum area; every wave takes the barrier
    constexpr int RED = 4 * TM * 16 * 64;  // floats of the partial-sum area
    uint32_t* xb = reinterpret_cast<uint32_t*>(smem) + RED;
    static_assert((RED + 2 * TM * 8 * 64) * 4 <= SMEM, "exchange buffer");
    const int wg = wn & 1;
    if (kh == 0 && wn >= 2 && nb >= 0) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int v = 0; v < 8; ++v) xb[((wg * TM + tm) * 8 + v) * 64 + lane] = swg[tm][v];
    }
    lds_barrier_plain();
    if (kh == 0 && wn < 2 && nb >= 0) {
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
            const uint32_t uw = xb[((wg * TM + tm) * 8 + 2 * q + h) * 64 + lane];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float gv = bf16_to_f32((uint16_t)(gw >> (16 * u)));
              const float uv = bf16_to_f32((uint16_t)(uw >> (16 * u)));
              av[2 * h + u] = gv / (1.0f + __expf(-gv)) * uv;
            }
          }
          *reinterpret_cast<uint2*>(p.act + (size_t)(pos0 + ml) * p.ldact + nb + 8 * q + 4 * g2) =
              make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
        }
      }
    }
  }
}

// Few tokens (M <= 64): the layer is a weight stream.  Workgroup: 8 waves,
// 128 channels x 64 tokens; wave (wn, kh) = (wave % 4, wave / 4) owns
// channels 32 wn + [0, 32), all 64 tokens, and the in-features of every
// other 64-wide step: a ring stage holds a 128-wide step, kh picks its half,
// so two waves share each SIMD and the two halves' partial sums are added
// in LDS at the end (fixed order).  Same copies, layouts, contraction order
// and epilogues as above (grouped: tiles of at most 64 expert positions;
// EPI_ROT_SWIGLU: 64 gate + 64 up channels per tile).  FP8: four stages,
// copies issued three 128-wide steps ahead; INT4: three stages (75 KB), two
// workgroups per CU, so that four waves per SIMD hide each other's waits.
// A tile of at most 32 rows skips the second token tile: its matrix work,
// and the activation copies of the waves whose rows all lie past row 31.
// BMD = 16 (INT4, grouped; experts of a few rows each): 16-row activation
// tiles (8 KB less per stage), so five stages (65 KB) fit, four 128-wide
// weight steps in flight per workgroup; the matrix cores see the 16 rows
// twice (token columns 16..31 are dropped).
namespace ntd {
constexpr int DEC_BN = 128, DEC_NST = 4, DEC_NTHR = 512;
template <bool FP8> constexpr int DEC_W_HALF = FP8 ? DEC_BN * BK : DEC_BN * BK / 2 + DEC_BN * 4;
}  // namespace ntd

template <int WF, int B, int EPI = EPI_ROT, bool GROUPED = false, int BMD = 64>
__global__ __launch_bounds__(ntd::DEC_NTHR, WF == WF_FP8 ? 1 : 2) void gemm_nt_dec_kernel(NtArgs p) {
  using namespace ntd;
  constexpr bool FP8 = WF == WF_FP8;
  static_assert(FP8 || wf_4bit(WF), "FP8 or 4-bit weights");
  static_assert(!wf_tiled(WF), "row-major weights only");
  static_assert(EPI == EPI_ROT || EPI == EPI_PLAIN || epi_swiglu(EPI) || EPI == EPI_BASE, "epilogue");
  static_assert(BMD == 64 || (BMD == 16 && !FP8 && GROUPED), "16-row tiles: grouped 4-bit weights");
  constexpr bool SWI = epi_swiglu(EPI);
  // INT4: three stages (75 KB; 16-row tiles: five, 65 KB), two workgroups
  // per CU; FP8: four stages
    constexpr int TM = BMD == 64 ? 2 : 1, NST = FP8 ? DEC_NST : (BMD == 16 ? 5 : DEC_NST - 1);
  constexpr int XI = BMD == 64 ? 2 : 1;  // activation copies per step of a copying wave
  constexpr int XH = BMD * BK * 2;      // 8 KB (2 KB): one 64-wide half of a step
  constexpr int WH = DEC_W_HALF<FP8>;   // weight bytes of one half
  constexpr int SB = 2 * XH + 2 * WH;   // stage bytes
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, kh = wave >> 2;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;
  int e = 0, pos0, nrows, cx = blockIdx.x;
  if constexpr (GROUPED) {
    int t;
    if (!grouped_tile(*p.ntiles, cx, t)) return;
    e = p.tiles[2 * t];
    pos0 = p.offsets[e] + p.tiles[2 * t + 1];
    nrows = min(BMD, p.offsets[e + 1] - pos0);
  } else {
    pos0 = blockIdx.y * BMD;
    nrows = min(BMD, p.M - pos0);
  }
  const uint8_t* wc = p.wc + (size_t)e * p.wc_e;
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws) + (size_t)e * p.ws_e;
  const uint16_t* rops = nt_rops(p) + (size_t)e * p.rops_e;
  // channel of local weight row rw (0..127), or -1 past the layer's channels
  const int cbase = SWI ? cx * (DEC_BN / 2) : cx * DEC_BN;
  auto chan = [&](int rw) -> int {
    if constexpr (SWI) {
      const int c = cbase + (rw & (DEC_BN / 2 - 1));
      return c < p.half_n ? (rw < DEC_BN / 2 ? c : p.half_n + c) : -1;
    } else {
      return cbase + rw < p.N ? cbase + rw : -1;
    }
  };
  auto crow = [&](int rw) { const int c = chan(rw); return c >= 0 ? c - cbase : 0; };
  const int nk = K / BK;          // 64-wide steps
  const int nk2 = (nk + 1) / 2;   // 128-wide steps
  const int kg = FP8 ? 1 : K / p.g;
  const int gs = p.g == 32 ? 1 : p.g == 64 ? 0 : -1;

  // copies of wave (wn, kh), for half kh of each step (a missing last half
  // re-copies the first half: same count, never read):
  //   activations rows 16 wn .. 16 wn + 15 (two instructions; 16-row
  //   tiles: rows 8 wn .. 8 wn + 7 on waves wn < 2, one instruction),
  //   weight rows 32 wn .. 32 wn + 31 (FP8: two instructions; INT4: one,
  //   plus the rows' scale words on lanes 0..31)
  const uint8_t* xbase = static_cast<const uint8_t*>(p.a) + (size_t)pos0 * p.lda * 2;
  uint32_t xoff[XI];
  const uint8_t* xptr[GROUPED ? XI : 1];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = (BMD == 64 ? 16 * wn + 8 * i : 8 * (wn & 1)) + (lane >> 3);
    const int rr = r < nrows ? r : 0;
    const int chunk = 16 * ((lane & 7) ^ swz_x(r));
    xoff[i] = (uint32_t)(rr * p.lda * 2 + chunk);
    if constexpr (GROUPED) {
      const long src = p.kslots > 0 ? (long)(p.perm[pos0 + rr] / p.kslots) : (long)(pos0 + rr);
      xptr[i] = static_cast<const uint8_t*>(p.a) + src * p.lda * 2 + chunk;
    }
  }
  const uint8_t* wbase = wc + (FP8 ? (size_t)cbase * K : (size_t)cbase * (K / 2));
  uint32_t woff[2] = {0u, 0u};
  uint32_t sbase = 0;
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rw = 32 * wn + 16 * i + (lane >> 2);
      woff[i] = (uint32_t)(crow(rw) * K + 16 * ((lane & 3) ^ swz_w8(rw)));
    }
  } else {
    const int rw = 32 * wn + (lane >> 1);
    woff[0] = (uint32_t)(crow(rw) * (K / 2) + 16 * ((lane & 1) ^ swz_w4(rw)));
    sbase = (uint32_t)((cbase + crow(32 * wn + l32)) * kg);
  }
  const uint32_t base_lds = lds_addr(smem);
  const uint32_t x_lds = base_lds + (uint32_t)(kh * XH + (BMD == 64 ? 16 * wn : 8 * (wn & 1)) * 128);
  const uint32_t w_lds = base_lds + (uint32_t)(2 * XH + kh * WH + 32 * wn * (FP8 ? 64 : 32));
  const uint32_t s_lds = base_lds + (uint32_t)(2 * XH + kh * WH + DEC_BN * BK / 2 + 32 * wn * 4);
  auto sstep = [&](int s) { return gs >= 0 ? s << gs : s >> 1; };

  // xc: this wave copies its activation rows (waves whose rows are all past
  // a tile of at most 32 rows skip them; their copy count per step is 2)
  auto issue = [&](int s2, bool xc) {  // 128-wide step s2, this wave's half
    const int st = s2 % NST;
    int s = 2 * s2 + kh;
    if (s >= nk) s = 2 * s2;
    const uint8_t* xb = xbase + (size_t)s * BK * 2;
    if (xc) {
#pragma unroll
      for (int i = 0; i < XI; ++i) {
        if constexpr (GROUPED)
          copy16v(x_lds + st * SB + 1024 * i, xptr[i] + (size_t)s * BK * 2);
        else
          copy16(x_lds + st * SB + 1024 * i, xb, xoff[i]);
      }
    }
    if constexpr (FP8) {
      const uint8_t* wb = wbase + (size_t)s * BK;
      copy16(w_lds + st * SB, wb, woff[0]);
      copy16(w_lds + st * SB + 1024, wb, woff[1]);
    } else {
      copy16(w_lds + st * SB, wbase + (size_t)s * (BK / 2), woff[0]);
      if (lane < 32) copy4(s_lds + st * SB, ws_h, ((sbase + (uint32_t)sstep(s)) * 2u) & ~3u);
    }
  };

  const int rw = 32 * wn + l32;  // this lane's operand row
  const int xsw = swz_x(l32);
  uint32_t wrd[2];
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) wrd[j] = (uint32_t)(rw * 64 + 16 * ((2 * g2 + j) ^ swz_w8(rw)));
  } else {
    wrd[0] = (uint32_t)(rw * 32 + 16 * (g2 ^ swz_w4(rw)));
    wrd[1] = 0u;
  }
  const uint32_t srd = FP8 ? 0u : (uint32_t)((cbase + crow(rw)) * kg);

  f32x16 acc[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;

  // TMV (a std::integral_constant): 32-token tiles that hold rows (1 when
  // the tile has at most 32 rows: the other tile is skipped)
  auto compute = [&](int s2, auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    const int s = 2 * s2 + kh;
    if (s >= nk) return;
    const int st = s2 % NST;
    const uint8_t* X = smem + st * SB + kh * XH;
    const uint8_t* W = smem + st * SB + 2 * XH + kh * WH;
    uint32_t cw[8];
    typename W4<WF>::S sc;
    if constexpr (FP8) {
      const uint4 c0 = *reinterpret_cast<const uint4*>(W + wrd[0]);
      const uint4 c1 = *reinterpret_cast<const uint4*>(W + wrd[1]);
      cw[0] = c0.x; cw[1] = c0.y; cw[2] = c0.z; cw[3] = c0.w;
      cw[4] = c1.x; cw[5] = c1.y; cw[6] = c1.z; cw[7] = c1.w;
    } else {
      const uint4 c0 = *reinterpret_cast<const uint4*>(W + wrd[0]);
      cw[0] = c0.x; cw[1] = c0.y; cw[2] = c0.z; cw[3] = c0.w;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(W + DEC_BN * BK / 2 + rw * 4);
      const uint32_t idx = srd + (uint32_t)(gs == 1 ? 2 * s + g2 : gs == 0 ? s : s >> 1);
      sc = W4<WF>::scale((uint16_t)(word >> (16 * (idx & 1))));
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a;
      if constexpr (FP8) {
        const uint2 lo = dq_fp8x4(cw[2 * kk]), hi = dq_fp8x4(cw[2 * kk + 1]);
        a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      } else {
        a = as_bf16x8(W4<WF>::dq(cw[kk], sc));
      }
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) {
        const int xr = BMD == 64 ? 32 * tm + l32 : (l32 & 15);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(X + xr * 128 + 16 * ((4 * g2 + kk) ^ xsw));
        acc[tm] = mfma32(a, b, acc[tm]);
      }
    }
  };

  auto run = [&](auto tmv_c) {
    constexpr int TMV = decltype(tmv_c)::value;
    const bool xc = BMD == 64 ? (TMV == 2 || wn < 2) : wn < 2;  // uniform
    const int per = (xc ? XI : 0) + 2;                          // copies per step of this wave
    const int pre = nk2 < NST - 1 ? nk2 : NST - 1;
    for (int s2 = 0; s2 < pre; ++s2) issue(s2, xc);
    for (int s2 = 0; s2 < nk2; ++s2) {
      // copies of steps s2 + 1 .. s2 + NST - 2 may stay in flight
      const int ahead = min(NST - 2, nk2 - 1 - s2);
      wait_copies_barrier_n(per * ahead);
      if (s2 + NST - 1 < nk2) issue(s2 + NST - 1, xc);
      compute(s2, tmv_c);
    }
  };
  if (BMD == 64 && nrows > 32)
    run(std::integral_constant<int, TM>{});
  else
    run(std::integral_constant<int, 1>{});

  dec_finish<FP8, B, EPI, TM, NST * SB>(p, acc, smem, wn, kh, lane, chan(32 * wn), nrows, pos0, rops);
}

// INT4 weight stream on 256-wide K steps (K % 256 == 0): every weight copy
// reads whole 128-byte lines (8 rows x 128 B per instruction), and a stage
// costs one barrier.  Workgroup: 8 waves, 128 channels x BMD tokens (16 or
// 64); wave (wn, kh) multiplies channels 32 wn + [0, 32) with in-features
// [128 kh, 128 kh + 128) of every step, the halves' partial sums are added
// at the end (dec_finish).  Stage (three, copies two steps ahead):
//   weights      128 rows x 128 B, chunk c of row r at c ^ ((r >> 1) & 7)
//   scales       128 rows x 512/g B
//   activations  BMD rows x 512 B, chunk c of row r at c ^ (r & 15)
// (16 consecutive rows read at one chunk hit 16 distinct 16-byte bank
// slots in both layouts).  16-row tiles: 78 KB, two workgroups per CU.
// Tiled INT4 storage (WF_INT4T, oft_formats.h): a step is two tile columns;
// the codes land as above, the scales as two halves (the step's two tiles)
// of 128 rows x 256/g bytes, copied 16 contiguous bytes a lane.
namespace ntd {
constexpr int D4_NST = 3;
}  // namespace ntd

template <int B, int EPI, bool GROUPED, int BMD, int WF = WF_INT4>
__global__ __launch_bounds__(ntd::DEC_NTHR, BMD == 16 ? 2 : 1) void gemm_nt_dec4_kernel(NtArgs p) {
  static_assert(wf_4bit(WF), "4-bit weights");
  using namespace ntd;
  static_assert(BMD == 16 || BMD == 64, "tile rows");
  static_assert(EPI == EPI_ROT || EPI == EPI_PLAIN || epi_swiglu(EPI) || EPI == EPI_BASE, "epilogue");
  constexpr bool SWI = epi_swiglu(EPI);
  constexpr bool TILED = wf_tiled(WF);
  constexpr int TM = BMD == 64 ? 2 : 1, NST = D4_NST;
  constexpr int WBY = 128 * 128, SBY = 128 * 16, XBY = BMD * 512, SB = WBY + SBY + XBY;
  constexpr int XI = BMD / 16;  // activation copies per wave per step (2 rows x 512 B each)
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, kh = wave >> 2;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;
  int e = 0, pos0, nrows, cx = blockIdx.x;
  if constexpr (GROUPED) {
    int t;
    if (!grouped_tile(*p.ntiles, cx, t)) return;
    e = p.tiles[2 * t];
    pos0 = p.offsets[e] + p.tiles[2 * t + 1];
    nrows = min(BMD, p.offsets[e + 1] - pos0);
  } else {
    pos0 = blockIdx.y * BMD;
    nrows = min(BMD, p.M - pos0);
  }
  const uint8_t* wc = p.wc + (size_t)e * p.wc_e;
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws) + (size_t)e * p.ws_e;
  const uint16_t* rops = nt_rops(p) + (size_t)e * p.rops_e;
  const int cbase = SWI ? cx * (DEC_BN / 2) : cx * DEC_BN;
  auto chan = [&](int rw) -> int {
    if constexpr (SWI) {
      const int c = cbase + (rw & (DEC_BN / 2 - 1));
      return c < p.half_n ? (rw < DEC_BN / 2 ? c : p.half_n + c) : -1;
    } else {
      return cbase + rw < p.N ? cbase + rw : -1;
    }
  };
  auto crow = [&](int rw) { const int c = chan(rw); return c >= 0 ? c - cbase : 0; };
  const int nks = K / 256;
  const int kg = K / p.g;
  const int sg = 512 / p.g;  // scale bytes per row and step: 16, 8 or 4
  // scale copy instructions per step: g = 64 takes four (two dwords a row);
  // tiled: 128 rows x 512/g bytes, 16 a lane (g = 32 two, else one)
  const int nsw = TILED ? (p.g == 32 ? 2 : 1) : p.g == 64 ? 4 : 2;

  // copies of wave w per step:
  //   weights rows 16 w + 8 i + lane / 8 (i = 0, 1), chunk lane % 8;
  //   activations rows 2 (XI w + i) + lane / 32, chunk lane % 32;
  //   scales (waves w < nsw): g = 32 16 B of row 64 w + lane; g = 64 dword
  //   64 w + lane (row / 2, half % 2); g = 128 the dword of row 64 w + lane.
  const uint8_t* wbase = wc + (size_t)cbase * (K / 2);
  uint32_t woff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rw = 16 * wave + 8 * i + (lane >> 3);
    const int cb = 16 * ((lane & 7) ^ ((rw >> 1) & 7));
    // (tiled: relative to the block of cbase, a multiple of 64)
    woff[i] = TILED ? t4_code_off(crow(rw), cb, K) : (uint32_t)(crow(rw) * (K / 2) + cb);
  }
  constexpr int WSTEP = TILED ? 2 * T4_TILE_BYTES : 128;  // code bytes from one step to the next
  uint32_t soff = 0;
  if constexpr (TILED) {
    // lane L = 64 wave + lane of the scale copies: half h (the step's tile
    // h), 64-row block j of the tile's 128 rows, 16-byte piece q of that
    // block's 64 x 256/g contiguous bytes; its LDS bytes are 16 L, i.e.
    // [half][row][256/g]
    const int sr = 256 / p.g;  // bytes a row in one tile
    const int L = 64 * wave + lane;
    const int h = L / (8 * sr), j = (L / (4 * sr)) & 1, q = L % (4 * sr);
    soff = t4_scale_off(crow(64 * j), 0, K, p.g) + (uint32_t)(h * (16384 / p.g) + 16 * q);
  } else {
    const int j = 64 * wave + lane;
    const int row = p.g == 64 ? (j >> 1) : j;
    const int sub = p.g == 64 ? 4 * (j & 1) : 0;
    soff = (uint32_t)((cbase + crow(row & 127)) * kg * 2 + sub);
  }
  const uint8_t* ws_b = reinterpret_cast<const uint8_t*>(ws_h) + (TILED ? (size_t)cbase * kg * 2 : 0);
  const int s_step = TILED ? 2 * 16384 / p.g : sg;  // scale bytes from one step to the next
  uint32_t xoff[XI];
  const uint8_t* xptr[GROUPED ? XI : 1];
  const uint8_t* xbase = static_cast<const uint8_t*>(p.a) + (size_t)pos0 * p.lda * 2;
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = 2 * (XI * wave + i) + (lane >> 5);
    const int rr = r < nrows ? r : 0;
    const int chunk = 16 * ((lane & 31) ^ (r & 15));
    xoff[i] = (uint32_t)(rr * p.lda * 2 + chunk);
    if constexpr (GROUPED) {
      const long src = p.kslots > 0 ? (long)(p.perm[pos0 + rr] / p.kslots) : (long)(pos0 + rr);
      xptr[i] = static_cast<const uint8_t*>(p.a) + src * p.lda * 2 + chunk;
    }
  }
  const uint32_t base_lds = lds_addr(smem);
  const uint32_t w_lds = base_lds + (uint32_t)(16 * wave * 128);
  const uint32_t s_lds = base_lds + (uint32_t)(WBY + (TILED ? 1024 * wave : p.g == 64 ? 4 * 64 * wave
                                                                           : (p.g == 32 ? 16 : 4) * 64 * wave));
  const uint32_t x_lds = base_lds + (uint32_t)(WBY + SBY + 2 * XI * wave * 512);
  const bool scopy = wave < nsw;
  const int per = 2 + XI + (scopy ? 1 : 0);  // copies per step of this wave

  auto issue = [&](int s) {
    const int st = s % NST;
    const uint32_t so = (uint32_t)(st * SB);
#pragma unroll
    for (int i = 0; i < 2; ++i) copy16(w_lds + so + 1024 * i, wbase + (size_t)s * WSTEP, woff[i]);
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      if constexpr (GROUPED)
        copy16v(x_lds + so + 1024 * i, xptr[i] + (size_t)s * 512);
      else
        copy16(x_lds + so + 1024 * i, xbase + (size_t)s * 512, xoff[i]);
    }
    if (scopy) {
      const uint8_t* sb = ws_b + (size_t)s * s_step;
      if (TILED) {
        if (p.g != 128 || lane < 32) copy16(s_lds + so, sb, soff);
      } else if (p.g == 32) {
        copy16(s_lds + so, sb, soff);
      } else {
        copy4(s_lds + so, sb, soff);
      }
    }
  };

  const int rw = 32 * wn + l32;  // this lane's operand row
  const int wsw = (rw >> 1) & 7;
  // activation chunk offsets of this lane (step-invariant): row xr, chunk
  // 16 kh + 8 g2 + kk; the second 32-row tile sits 32 rows (16 KB) further
  const int xr0 = BMD == 64 ? l32 : (l32 & 15);
  uint32_t xo[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) xo[kk] = (uint32_t)(xr0 * 512 + 16 * ((16 * kh + 8 * g2 + kk) ^ (xr0 & 15)));
  f32x16 acc[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;

  auto compute = [&](auto tmv_c, auto st_c) {  // st_c: the ring stage, a constant
    constexpr int TMV = decltype(tmv_c)::value;
    const uint8_t* W = smem + decltype(st_c)::value * SB;
    const uint8_t* S = W + WBY;
    const uint8_t* X = S + SBY;
    const int c0 = 4 * kh + 2 * g2;  // this lane's two 16-byte chunks: in-features 32 c0 .. 32 c0 + 63
    const uint4 v0 = *reinterpret_cast<const uint4*>(W + rw * 128 + 16 * (c0 ^ wsw));
    const uint4 v1 = *reinterpret_cast<const uint4*>(W + rw * 128 + 16 * ((c0 + 1) ^ wsw));
    uint32_t sw;
    if (TILED) {
      // half kh (in-features 128 kh + ...), this lane's slots 64 g2 / g of it
      const int sr = 256 / p.g;
      const uint8_t* sp = S + kh * 128 * sr + rw * sr;
      if (p.g == 32)
        sw = *reinterpret_cast<const uint32_t*>(sp + 4 * g2);
      else
        sw = *reinterpret_cast<const uint16_t*>(sp + (p.g == 64 ? 2 * g2 : 0));
    } else if (p.g == 32) {
      sw = *reinterpret_cast<const uint32_t*>(S + rw * 16 + 2 * c0);
    } else {
      sw = *reinterpret_cast<const uint16_t*>(S + rw * sg + 2 * (p.g == 64 ? c0 / 2 : kh));
    }
    // every activation operand of the step is read before the first
    // dequantisation, so the LDS latency is paid once per step
    bf16x8 xb[8][TMV];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) xb[kk][tm] = *reinterpret_cast<const bf16x8*>(X + xo[kk] + 16384 * tm);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t cw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    typename W4<WF>::S sc[2];
    sc[0] = W4<WF>::scale((uint16_t)sw);
    sc[1] = p.g == 32 ? W4<WF>::scale((uint16_t)(sw >> 16)) : sc[0];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 a = as_bf16x8(W4<WF>::dq(cw[kk], sc[kk >> 2]));
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) acc[tm] = mfma32(a, xb[kk][tm], acc[tm]);
    }
  };

  auto run = [&](auto tmv_c) {
    const int pre = nks < NST - 1 ? nks : NST - 1;
    for (int s = 0; s < pre; ++s) issue(s);
    ring_steps<NST>(nks, [&](int s, auto st_c) {
      // copies of steps s + 1 .. s + NST - 2 may stay in flight
      const int ahead = min(NST - 2, nks - 1 - s);
      wait_copies_barrier_n(per * ahead);
      if (s + NST - 1 < nks) issue(s + NST - 1);
      compute(tmv_c, st_c);
    });
  };
  if (BMD == 64 && nrows > 32)
    run(std::integral_constant<int, TM>{});
  else
    run(std::integral_constant<int, 1>{});

  dec_finish<false, B, EPI, TM, NST * SB>(p, acc, smem, wn, kh, lane, chan(32 * wn), nrows, pos0, rops);
}


// Dense decode (M <= 64 tokens, 4-bit weights, K % 256 == 0): the same
// stage layout, copies and channel tile (128) as gemm_nt_dec4_kernel, with
// sixteen waves per workgroup, four per SIMD: wave (wn, kq) = (wave % 4,
// wave / 4) multiplies channels 32 wn + [0, 32) with in-features
// [64 kq, 64 kq + 64) of every 256-wide step (one 16-byte chunk of codes per
// lane, four matrix steps), so each SIMD has four independent instruction
// streams to overlap dequantisation, matrix work and LDS reads, and the
// four parts' sums are added in part order at the end (dec_finish).  Every
// wave issues the same copies each step (one weight, two activation, and
// for the first two or four waves one scale copy), so the waits are
// compile-time counts.
template <int B, int EPI, int WF = WF_INT4>
__global__ __launch_bounds__(1024, 1) void gemm_nt_dec16_kernel(NtArgs p) {
  static_assert(wf_4bit(WF) && !wf_tiled(WF), "row-major 4-bit weights");
  static_assert(EPI == EPI_ROT || EPI == EPI_PLAIN || EPI == EPI_BASE, "epilogue");
  using namespace ntd;
  constexpr int NST = 3, BMD = 64, TM = 2;
  constexpr int WBY = 128 * 128, SBY = 128 * 16, XBY = BMD * 512, SB = WBY + SBY + XBY;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3, kq = wave >> 2;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;
  const int nrows = min(BMD, p.M);
  const uint8_t* wc = p.wc;
  const uint16_t* ws_h = static_cast<const uint16_t*>(p.ws);
  const uint16_t* rops = nt_rops(p);
  const int cbase = blockIdx.x * DEC_BN;
  auto chan = [&](int rw) -> int { return cbase + rw < p.N ? cbase + rw : -1; };
  auto crow = [&](int rw) { const int c = chan(rw); return c >= 0 ? c - cbase : 0; };
  const int nks = K / 256;
  const int kg = K / p.g;
  const int sg = 512 / p.g;  // scale bytes per row and step: 16, 8 or 4
  const int nsw = p.g == 64 ? 4 : 2;

  // copies of wave w per step: weight rows 8 w + lane / 8, chunk lane % 8
  // (one instruction); activation rows 4 w + 2 i + lane / 32 (i = 0, 1),
  // chunk lane % 32; scales as in gemm_nt_dec4_kernel (waves w < nsw)
  const uint8_t* wbase = wc + (size_t)cbase * (K / 2);
  uint32_t woff;
  {
    const int rw = 8 * wave + (lane >> 3);
    woff = (uint32_t)(crow(rw) * (K / 2) + 16 * ((lane & 7) ^ ((rw >> 1) & 7)));
  }
  uint32_t soff = 0;
  {
    const int j = 64 * (wave < nsw ? wave : 0) + lane;
    const int row = p.g == 64 ? (j >> 1) : j;
    const int sub = p.g == 64 ? 4 * (j & 1) : 0;
    soff = (uint32_t)((cbase + crow(row & 127)) * kg * 2 + sub);
  }
  uint32_t xoff[2];
  const uint8_t* xbase = static_cast<const uint8_t*>(p.a);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * wave + 2 * i + (lane >> 5);
    const int rr = r < nrows ? r : 0;
    xoff[i] = (uint32_t)(rr * p.lda * 2 + 16 * ((lane & 31) ^ (r & 15)));
  }
  const uint32_t base_lds = lds_addr(smem);
  const uint32_t w_lds = base_lds + (uint32_t)(1024 * wave);
  const uint32_t s_lds = base_lds + (uint32_t)(WBY + (p.g == 64 ? 4 * 64 * wave : (p.g == 32 ? 16 : 4) * 64 * wave));
  const uint32_t x_lds = base_lds + (uint32_t)(WBY + SBY + 2048 * wave);

  auto issue = [&](int s, auto sc_c) {
    constexpr bool SC = decltype(sc_c)::value;
    const uint32_t so = (uint32_t)((s % NST) * SB);
    copy16(w_lds + so, wbase + (size_t)s * 128, woff);
#pragma unroll
    for (int i = 0; i < 2; ++i) copy16(x_lds + so + 1024 * i, xbase + (size_t)s * 512, xoff[i]);
    if constexpr (SC) {
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(ws_h) + (size_t)s * sg;
      if (p.g == 32)
        copy16(s_lds + so, sb, soff);
      else
        copy4(s_lds + so, sb, soff);
    }
  };

  const int rw = 32 * wn + l32;  // this lane's operand row
  const int cq = 2 * kq + g2;    // this lane's 16-byte code chunk of the step: in-features 32 cq .. 32 cq + 31
  const uint32_t w_rd = (uint32_t)(rw * 128 + 16 * (cq ^ ((rw >> 1) & 7)));
  const uint32_t s_rd = (uint32_t)(WBY + (p.g == 32 ? rw * 16 + 2 * cq : rw * sg + 2 * (p.g == 64 ? kq : kq >> 1)));
  uint32_t xo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) xo[kk] = (uint32_t)(WBY + SBY + l32 * 512 + 16 * ((4 * cq + kk) ^ (l32 & 15)));
  f32x16 acc[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;

  auto compute = [&](auto tmv_c, auto st_c) {  // st_c: the ring stage, a constant
    constexpr int TMV = decltype(tmv_c)::value;
    const uint8_t* St = smem + decltype(st_c)::value * SB;
    const uint4 cw4 = *reinterpret_cast<const uint4*>(St + w_rd);
    const uint16_t sbits = *reinterpret_cast<const uint16_t*>(St + s_rd);
    // every activation operand of the step is read before the first
    // dequantisation, so the LDS latency is paid once per step
    bf16x8 xb[4][TMV];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) xb[kk][tm] = *reinterpret_cast<const bf16x8*>(St + xo[kk] + 16384 * tm);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t cw[4] = {cw4.x, cw4.y, cw4.z, cw4.w};
    const typename W4<WF>::S sc = W4<WF>::scale(sbits);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = as_bf16x8(W4<WF>::dq(cw[kk], sc));
#pragma unroll
      for (int tm = 0; tm < TMV; ++tm) acc[tm] = mfma32(a, xb[kk][tm], acc[tm]);
    }
  };

  auto run = [&](auto tmv_c, auto sc_c) {
    constexpr int PER = 3 + (decltype(sc_c)::value ? 1 : 0);  // copies per step of this wave
    const int pre = nks < NST - 1 ? nks : NST - 1;
    for (int s = 0; s < pre; ++s) issue(s, sc_c);
    ring_steps<NST>(nks, [&](int s, auto st_c) {
      // the copies of step s + 1 may stay in flight
      if (s + 1 < nks)
        wait_copies_barrier_n(PER);
      else
        wait_copies_barrier_n(0);
      if (s + NST - 1 < nks) issue(s + NST - 1, sc_c);
      compute(tmv_c, st_c);
    });
  };
  if (nrows > 32) {
    if (wave < nsw)
      run(std::integral_constant<int, TM>{}, std::true_type{});
    else
      run(std::integral_constant<int, TM>{}, std::false_type{});
  } else {
    if (wave < nsw)
      run(std::integral_constant<int, 1>{}, std::true_type{});
    else
      run(std::integral_constant<int, 1>{}, std::false_type{});
  }

  dec_finish<false, B, EPI, TM, NST * SB, 4>(p, acc, smem, wn, kq, lane, chan(32 * wn), nrows, 0, rops);
}

}  // namespace oft
