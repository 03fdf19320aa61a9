// Backward-type 4-bit dequant GEMM on the copy ring:
//   C^T[k][m] = sum_n W[n][k] B[m][n]
// the product of gemm_nn_dma.h (the contraction runs over the weight's rows
// n, the weight as stored, no transposed copy), for INT4 weights with fp16
// group scales along k; B rows are bf16, dense rows or gathered expert
// positions (kslots > 0: row perm[pos] / kslots); epilogues EPI_STORE and
// EPI_SWIGLU_BWD of gemm_nn.h (bf16 out).  The host guarantees K % 256 == 0
// and N % 64 == 0.
//
// Workgroup: 8 waves, tile 256 output columns x 128 rows, contraction steps
// of 64 weight rows.  Wave w owns columns 32 w + [0, 32) of the tile, which
// lie in one scale group, and every row (four 32-row matrix-core tiles,
// skipped past the tile's last row); so every weight code of the tile is
// dequantised by one wave only.
//
// Every HBM read of the main loop is a global_load_lds copy, counted by the
// kernel itself (vmcnt) as in gemm_nt_dma.h, through three LDS stages issued
// two steps ahead:
//   B      : 128 rows x 128 B, 16-byte piece p of row r at p ^ swz_x(r)
//            (two copies per wave; copies holding no row of the tile are
//            skipped);
//   codes  : 64 rows n x 128 B (the tile's 256 columns, two per byte), piece
//            p of row n at p ^ ((n >> 1) & 7) (one copy per wave: its 8 rows);
//   scales : wave w's 64 dwords, dword j = s[n0 + j][group of the wave's
//            columns] (global_load_lds_ushort puts lane j's two bytes in
//            the low half of LDS dword j), one copy per wave.
//
// Matrix-core operands (v_mfma_f32_32x32x16_bf16): A = W^T, rows = the
// wave's 32 columns, contraction along n, read with the gfx950 4-bit
// transpose load ds_read_b64_tr_b4: within each 16-lane group, output lane
// 16G + r receives nibble r of the 8-byte pieces read by lanes 16G + e as
// its nibble e (e = 0..15; probed).  Pointing lane 16G + e at row
// n0 + 16 (G >> 1) + e, columns 32 w + 16 (G & 1) + [0, 16) gives lane
// (l32, g2) the codes W[n0 + 16 g2 + e][32 w + l32], e = 0..15; the XOR
// swizzle of the code rows spreads those 16 rows over all 64 LDS banks.
// Each code is dequantised in registers with the scale of its own row n:
// bf16(q s), q from the fp16 1024 + (nibble ^ 8) minus 1032 (exact), the
// product exact in fp32, one rounding: the dequant hook's value.  In MFMA
// kk (0..3) of a step, lane group g2 takes the contraction indices
// 32 (kk >> 1) + 16 g2 + 8 (kk & 1) + p (p = 0..7) for both operands.
//
// TILED: the weight in the tiled INT4 storage of oft_formats.h.  A step's
// 64 weight rows are one 64-row block, its 256 columns two tile columns, so
// the codes land in the same LDS layout from two 4 KB tiles (each wave's 8
// rows: 256 contiguous bytes per tile quarter) and the 64 scales of a wave
// are 64 slots 256/g bytes apart in one tile (row-major: 64 rows apart).
#pragma once

#include <type_traits>

#include "gemm_nn.h"
#include "gemm_nt_dma.h"

namespace oft {

namespace nnq {
constexpr int BKO = 256;                 // output columns per workgroup
constexpr int BNS = 64;                  // weight rows per step
constexpr int BM = 128;                  // rows (tokens / positions)
constexpr int NTHR = 512;
constexpr int NST = 3;                   // ring depth
constexpr int B_BYTES = BM * BNS * 2;    // B tile
constexpr int C_BYTES = BNS * BKO / 2;   // codes
constexpr int S_BYTES = 8 * BNS * 4;     // scales (dword slots)
constexpr int STAGE = B_BYTES + C_BYTES + S_BYTES;
__device__ __forceinline__ int swz_c(int n) { return (n >> 1) & 7; }

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
__device__ __forceinline__ uint2 ds_read_tr4(const uint8_t* p) {
  const v2i v = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_v2i*)p);
  return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}

// 8 INT4 codes (low nibble first) with one fp16 scale each (sc[e]: the fp16
// bits in the low half) -> 8 bf16, each bf16(q s) rounded once.  One AND/XOR
// per two nibbles puts them in fp16 mantissas with the nibble's top bit
// flipped (n ^ 8 = q + 8): nibbles in bits 0-3 of a half under exponent 10
// (value 1024 + (q + 8)), nibbles in bits 4-7 under exponent 6, whose unit
// is then the mantissa's bit 4 (value 64 + (q + 8)); so one shift by 8 bits
// serves all eight.  Subtracting 1032 or 72 (two at a time, packed fp16,
// exact) gives q, and one mixed fp16 x fp16 + fp32 FMA with a zero addend
// gives q s exactly in fp32 (at most 15 significant bits).  The zero addend
// turns a -0 product into +0, which no product of the matrix cores can tell
// apart.
__device__ __forceinline__ uint4 dq_i4x8_rows(uint32_t w, const uint32_t* sc) {
  const uint32_t v[2] = {w, w >> 8};
  float f[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f16x2 lo = __builtin_bit_cast(f16x2, (v[j] & 0x000F000Fu) ^ 0x64086408u);  // nibbles 2j, 2j + 4
    f16x2 hi = __builtin_bit_cast(f16x2, (v[j] & 0x00F000F0u) ^ 0x54805480u);  // nibbles 2j + 1, 2j + 5
    const f16x2 olo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2 ohi = {(_Float16)-72.0f, (_Float16)-72.0f};
    lo = lo + olo;
    hi = hi + ohi;
    f[2 * j] = __builtin_fmaf((float)lo[0], (float)__builtin_bit_cast(_Float16, (uint16_t)sc[2 * j]), 0.0f);
    f[2 * j + 4] = __builtin_fmaf((float)lo[1], (float)__builtin_bit_cast(_Float16, (uint16_t)sc[2 * j + 4]), 0.0f);
    f[2 * j + 1] = __builtin_fmaf((float)hi[0], (float)__builtin_bit_cast(_Float16, (uint16_t)sc[2 * j + 1]), 0.0f);
    f[2 * j + 5] = __builtin_fmaf((float)hi[1], (float)__builtin_bit_cast(_Float16, (uint16_t)sc[2 * j + 5]), 0.0f);
  }
  uint4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}
}  // namespace nnq

template <int EPI, bool GROUPED, bool TILED = false>
__global__ __launch_bounds__(nnq::NTHR, 2) void gemm_nn_q4_kernel(NnArgs p) {
  using namespace nnq;
  using ntd::copy16;
  using ntd::copy2;
  using ntd::copy16v;
  using ntd::lds_addr;
  using ntd::swz_x;
  static_assert(EPI == EPI_STORE || EPI == EPI_SWIGLU_BWD, "epilogue");
  static_assert(NST * STAGE <= 80 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int K = p.K;
  // contraction split (dense, few rows: nsplit_len > 0, a multiple of BNS):
  // workgroup z covers weight rows [z nsplit_len, (z + 1) nsplit_len) and
  // stores fp32 partials to part[z][M][K]
  const int zlo = (!GROUPED && p.nsplit_len > 0) ? (int)blockIdx.z * p.nsplit_len : 0;
  const int ns = (!GROUPED && p.nsplit_len > 0) ? min(p.nsplit_len, p.N - zlo) / BNS : p.N / BNS;

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
  const int kg = K / p.g;                // scales per weight row
  const uint8_t* wc = p.wc + (size_t)e * p.wc_e + (size_t)zlo * (K / 2);
  const uint8_t* ws_b = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(p.ws) + (size_t)e * p.ws_e +
                                                         (size_t)zlo * kg);
  const int gw = (kbase + 32 * wave) / p.g;  // scale group of this wave's columns

  // ---- B tile copies: rows 16 wave + 8 i + lane / 8 (past the end: row 0)
  const uint8_t* bbase = reinterpret_cast<const uint8_t*>(p.src) + ((size_t)pos0 * p.lds + zlo) * 2;
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
  // B copies of this wave that hold a row of the tile (the rest would only
  // copy rows past its end, whose products are never stored: skipped)
  const int vb = (16 * wave < nrows ? 1 : 0) + (16 * wave + 8 < nrows ? 1 : 0);
  const int vw = vb + 2;  // copies per step of this wave: B, codes, scales

  // ---- code copy: rows n = 8 wave + lane / 8, LDS piece lane % 8 holds
  // global piece (lane % 8) ^ swz_c(n) of the row's 128 bytes
  // (the step's rows n0 = 64 s: a whole block of the tiled layout, which
  // starts where row n0 does in the row-major one)
  const int cn = 8 * wave + (lane >> 3);
  const int cbyte = kbase / 2 + 16 * ((lane & 7) ^ swz_c(cn));
  const uint32_t coff = TILED ? oft::t4_code_off(cn, cbyte, K) : (uint32_t)(cn * (K / 2) + cbyte);
  // scale copy: lane j -> s[n0 + j][gw]
  const uint32_t soff = TILED ? oft::t4_scale_off(lane, gw, K, p.g) : (uint32_t)((lane * kg + gw) * 2);

  const uint32_t base_lds = lds_addr(smem);
  auto issue = [&](int s) {
    const uint32_t st = base_lds + (uint32_t)((s % NST) * STAGE);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= vb) break;
      if constexpr (GROUPED)
        copy16v(st + 16 * wave * 128 + i * 1024, bptr[i] + (size_t)s * BNS * 2);
      else
        copy16(st + 16 * wave * 128 + i * 1024, bbase + (size_t)s * BNS * 2, boff[i]);
    }
    copy16(st + B_BYTES + 1024 * wave, wc + (size_t)s * BNS * (K / 2), coff);
    copy2(st + B_BYTES + C_BYTES + 256 * wave, ws_b + (size_t)s * BNS * kg * 2, soff);
  };

  // ---- operand addresses (bytes within a stage)
  const int G = lane >> 4, er = lane & 15;
  const int an = 16 * (G >> 1) + er;  // code row of this lane's transpose piece (half 0)
  const uint32_t ard = (uint32_t)(B_BYTES + an * 128 + 16 * (wave ^ swz_c(an)) + 8 * (G & 1));
  const uint32_t srd = (uint32_t)(B_BYTES + C_BYTES + 256 * wave + 4 * 16 * g2);
  const int xsw = swz_x(l32);
  uint32_t brd[4];
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) brd[tm] = (uint32_t)((32 * tm + l32) * 128);

  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;

  // TMV (a std::integral_constant): 32-row tiles that hold rows; ST: the
  // ring stage of step s (s % NST), a constant so that the stage offset is
  // the LDS reads' immediate rather than per-address arithmetic
  auto compute = [&](auto tmv_c, auto st_c) {
    constexpr int TMV = decltype(tmv_c)::value, ST = decltype(st_c)::value;
    if constexpr (TMV > 0) {
      const uint8_t* S = smem + ST * STAGE;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // codes of rows 32 hf + 16 g2 + [0, 16) of the lane's column, and
        // their scales (dwords 32 hf + 16 g2 + [0, 16) of the wave's slots)
        const uint2 cw = ds_read_tr4(S + ard + hf * 32 * 128);
        uint32_t sc[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = *reinterpret_cast<const uint4*>(S + srd + hf * 128 + 16 * q);
          sc[4 * q] = v.x;
          sc[4 * q + 1] = v.y;
          sc[4 * q + 2] = v.z;
          sc[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const bf16x8 a = as_bf16x8(dq_i4x8_rows(sub ? cw.y : cw.x, sc + 8 * sub));
          const int piece = 4 * hf + 2 * g2 + sub;
#pragma unroll
          for (int tm = 0; tm < TMV; ++tm) {
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(S + brd[tm] + 16 * (piece ^ xsw));
            acc[tm] = mfma32(a, b, acc[tm]);
          }
        }
      }
    }
  };

  // every wave takes the same barriers, whatever its TMV; the step loop is
  // unrolled by the ring depth
  static_assert(NST == 3, "two steps of copies in flight");
  auto run = [&](auto tmv_c) {
    issue(0);
    if (ns > 1) issue(1);
    ring_steps<NST>(ns, [&](int s, auto st_c) {
      // copies of step s + 1 may stay in flight
      ntd::wait_copies_barrier_n(s + 1 < ns ? vw : 0);
      if (s + 2 < ns) issue(s + 2);
      compute(tmv_c, st_c);
    });
  };
  if (nrows > 96)
    run(std::integral_constant<int, 4>{});
  else if (nrows > 64)
    run(std::integral_constant<int, 3>{});
  else if (nrows > 32)
    run(std::integral_constant<int, 2>{});
  else
    run(std::integral_constant<int, 1>{});

  // ------------------------------------------------------------ epilogue
  // lane (l32, g2) holds, for row m = 32 tm + l32, columns
  // kbase + 32 wave + 8 q + 4 g2 + [0, 4) in registers 4 q .. 4 q + 3
  const int kb = kbase + 32 * wave;
  if constexpr (EPI == EPI_STORE) {
    const bool split = !GROUPED && p.nsplit_len > 0;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
      const int ml = 32 * tm + l32;
      if (ml >= nrows) continue;
      const f32x16& o = acc[tm];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t off = (size_t)(pos0 + ml) * p.ldo + kb + 8 * q + 4 * g2;
        if (split)
          *reinterpret_cast<float4*>(p.part + (size_t)blockIdx.z * p.M * p.ldo + off) =
              make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        else
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) =
              make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
      }
    }
  } else {
    // SwiGLU backward; out = dH [P, 2I] with ldo, K = I (see gemm_nn.h)
    float dwp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
      const int ml = 32 * tm + l32;
      if (ml >= nrows) continue;
      const long pos = (long)(pos0 + ml);
      const float wgt = p.topk_w[p.perm[pos]];
      const f32x16& o = acc[tm];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = kb + 8 * q + 4 * g2;
        const uint2 hg = *reinterpret_cast<const uint2*>(p.hsave + pos * p.ldh + col);
        const uint2 hu = *reinterpret_cast<const uint2*>(p.hsave + pos * p.ldh + K + col);
        const uint32_t gwd[2] = {hg.x, hg.y}, uwd[2] = {hu.x, hu.y};
        float dg[4], du[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float gv = bf16_to_f32((uint16_t)(gwd[s >> 1] >> (16 * (s & 1))));
          const float uv = bf16_to_f32((uint16_t)(uwd[s >> 1] >> (16 * (s & 1))));
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
    // per-row partial of dw over the tile's 256 columns: the two lane
    // halves, then the eight waves in order (fixed-order sums)
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) dwp[tm] += __shfl_xor(dwp[tm], 32);
    ntd::lds_barrier_plain();  // the ring is no longer read: it holds the partials
    float* red = reinterpret_cast<float*>(smem);
    if (g2 == 0) {
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) red[wave * BM + 32 * tm + l32] = dwp[tm];
    }
    __syncthreads();
    if (tid < BM && tid < nrows) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) sum += red[w * BM + tid];
      p.dw_part[(size_t)cx * p.P + pos0 + tid] = sum;
    }
  }
}

}  // namespace oft
