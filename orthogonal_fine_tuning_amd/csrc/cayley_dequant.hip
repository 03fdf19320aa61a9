// Cayley build (adapter parameters -> block rotations) and the dequant hook.
//
// Cayley map: the Orbit pages (chooseai.io release news, "Technical
// principles" and "Architectural advantages of OFT over LoRA") make every
// sub-projection's rotation orthogonal; this library builds each b x b block
// as R = (I + Q)(I - Q)^-1 = 2 (I - Q)^-1 - I from the skew-symmetric Q.
//
// Layout of the solve: in-place Gauss-Jordan on A = I - Q with row
// ownership (the in-place form keeps the growing inverse in the columns
// already eliminated).  Many blocks: a block per 16-lane row of a wave, each
// lane holding b / 16 rows of A in registers; a pivot step broadcasts the
// pivot row from its owner lane by DPP and every lane applies one fused
// multiply-add per element it holds.  Few blocks (a dense layer's build):
// two lanes per row, the pivot row published through LDS.  No pivot search
// is needed: the symmetric part of A is I, so every pivot is >= 1.
#include <utility>

#include "oft_device.h"
#include "oft_launch.h"
#include "oft_prof.h"

namespace oft {

// LDS hand-off among the lanes of one wave (the workgroup is one wave): a
// wavefront-scope release / acquire pair.  The LDS of a wave executes its
// operations in issue order, so this orders the accesses for the compiler
// without waiting for the writes to complete.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// f(integral_constant<int, S>) for S in order
template <class F, int... S>
__device__ __forceinline__ void for_each_index(F& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}

// value x of lane n of this lane's 16-lane row (DPP row_newbcast)
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(N >= 0 && N < 16, "row lane");
  // (every lane's source exists, so bound_ctrl changes nothing; with it
  // the move needs no old value)
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, true));
}

// A block per 16-lane row of the wave (four per wave): lane (sub, qd), qd =
// lane % 16, holds rows qd + 16 t (t = 0 .. RPL - 1, RPL = B / 16) of block
// blk0 + sub.  A pivot step broadcasts each element of the pivot row from
// its owner lane to the row by DPP (row_newbcast) just before the
// multiply-adds that use it, so the step loop touches no LDS and needs no
// synchronisation; each element sees the same operations in the same order
// as with any other row ownership.
template <int B>
__global__ __launch_bounds__(64) void cayley_kernel(const uint16_t* __restrict__ q, int nblk,
                                                    float* __restrict__ Rf, uint16_t* __restrict__ Rops) {
  constexpr int LPB = 16;         // lanes per block: one DPP row
  constexpr int RPL = B / LPB;    // rows per lane
  constexpr int PER = 64 / LPB;   // blocks per wave
  constexpr int NP = B * (B - 1) / 2;
  // the parameters of the wave's blocks, later the outputs of BR blocks at
  // a time: R in fp32 rows of FP floats, then R and R^T in bf16 rows of OP
  constexpr int BR = B == 32 ? 2 : 4;
  constexpr int FP = B + 4, OP = B + 8;  // (pitches: 16-byte rows, spread banks)
  constexpr int S_Q = PER * NP * 4, S_F = BR * B * FP * 4, S_O = BR * 2 * B * OP * 2;
  constexpr int STAGE = S_Q > S_F ? (S_Q > S_O ? S_Q : S_O) : (S_F > S_O ? S_F : S_O);
  static_assert(PER % BR == 0 && (BR * B * B / 4) % 64 == 0, "store rounds");
  __shared__ __attribute__((aligned(16))) uint8_t stage[STAGE];

  const int lane = threadIdx.x;
  const int sub = lane / LPB, qd = lane % LPB;
  const int blk0 = blockIdx.x * PER;
  const int nv = min(PER, nblk - blk0);  // blocks of this wave
  // parameters: PER consecutive blocks are PER * NP contiguous bf16; every
  // load of the wave is in flight before the first is used
  float* qs = reinterpret_cast<float*>(stage);
  const uint16_t* qw = q + (size_t)blk0 * NP;
  const int nq = nv * NP;
  static_assert(NP % 8 == 0, "whole 16-byte chunks per block");
  if ((reinterpret_cast<uintptr_t>(q) & 15) == 0) {  // then so is every wave's span
    constexpr int NV = (PER * NP / 8 + 63) / 64;
    uint4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int idx = lane + 64 * k;
      v[k] = reinterpret_cast<const uint4*>(qw)[min(idx, nq / 8 - 1)];  // clamped: no branch
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int idx = lane + 64 * k;
      if (8 * idx < nq) {
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          qs[8 * idx + 2 * t] = __uint_as_float(w[t] << 16);
          qs[8 * idx + 2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
        }
      }
    }
  } else {
    constexpr int NV = (PER * NP + 63) / 64;
    uint16_t v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = qw[min(lane + 64 * k, nq - 1)];  // clamped: no branch
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (lane + 64 * k < nq) qs[lane + 64 * k] = bf16_to_f32(v[k]);
  }
  __syncthreads();

  // A[r][c] = delta_rc - Q[r][c], Q[r][c] = p(r, c) above the diagonal and
  // -p(c, r) below (row-major upper-triangle order of p)
  float a[RPL][B];
  const float* qb = qs + sub * NP;
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int r = qd + LPB * t;
#pragma unroll
    for (int c = 0; c < B; ++c) {
      const int lo = c < r ? c : r, hi = c < r ? r : c;
      const float v = (c == r || sub >= nv) ? 0.0f : qb[lo * B - lo * (lo + 1) / 2 + (hi - lo - 1)];
      a[t][c] = c == r ? 1.0f : (c > r ? -v : v);
    }
  }
  __syncthreads();  // stage is reused for the outputs at the end

  // one pivot step; the step index is a compile-time constant so that every
  // a[][] access stays a register and the owner lane is the DPP operand
  auto step = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int ts = s / LPB, own = s % LPB;  // the pivot row: slot ts of lane own
    const bool owner = qd == own;
    // 1 / pivot: hardware reciprocal and one Newton step
    const float piv = row_bcast<own>(a[ts][s]);
    float rp = __builtin_amdgcn_rcpf(piv);
    rp = fmaf(rp, fmaf(-piv, rp, 1.0f), rp);
    // pivot row: a_sj / p; other rows: a_rj - (a_rs / p) a_sj; column s of
    // the inverse: 1 / p on the pivot row, -a_rs / p elsewhere.  Each pivot
    // element is taken from its owner before any update of its column.
    float g[RPL];
#pragma unroll
    for (int t = 0; t < RPL; ++t) g[t] = (t == ts && owner) ? 1.0f - rp : a[t][s] * rp;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (j == s) continue;
      const float pj = row_bcast<own>(a[ts][j]);
#pragma unroll
      for (int t = 0; t < RPL; ++t) a[t][j] = fmaf(-g[t], pj, a[t][j]);
    }
#pragma unroll
    for (int t = 0; t < RPL; ++t) a[t][s] = (t == ts && owner) ? rp : -g[t];
  };
  for_each_index(step, std::make_integer_sequence<int, B>{});

  // row r = qd + LPB t of A^-1 in a[t]; R = 2 A^-1 - I
#pragma unroll
  for (int t = 0; t < RPL; ++t)
#pragma unroll
    for (int j = 0; j < B; ++j) a[t][j] = 2.0f * a[t][j] - (j == qd + LPB * t ? 1.0f : 0.0f);
  // The outputs leave through LDS, BR blocks at a time, so that every store
  // instruction writes 64 consecutive 16-byte pieces (a block's R, and its
  // R | R^T pack, are contiguous; rows written straight from the lanes that
  // hold them would be 16-byte pieces of 64 rows)
  float* F = reinterpret_cast<float*>(stage);         // [BR][B][FP] fp32
  uint16_t* O = reinterpret_cast<uint16_t*>(stage);   // [BR][2][B][OP] bf16: R, R^T
#pragma unroll
  for (int rd = 0; rd < PER / BR; ++rd) {
    const int bb = sub - BR * rd;  // this lane's block in the round, if 0 <= bb < BR
    __syncthreads();  // the stage is free (parameters read, or the last round stored)
    if (bb >= 0 && bb < BR) {
#pragma unroll
      for (int t = 0; t < RPL; ++t)
#pragma unroll
        for (int j = 0; j < B; j += 4)
          *reinterpret_cast<float4*>(F + (bb * B + qd + LPB * t) * FP + j) =
              make_float4(a[t][j], a[t][j + 1], a[t][j + 2], a[t][j + 3]);
    }
    __syncthreads();
#pragma unroll 2  // (the rows in registers are still live: few loads in flight)
    for (int i = 0; i < BR * B * B / 4 / 64; ++i) {
      const int c = lane + 64 * i, cb = c / (B * B / 4), rem = c % (B * B / 4);
      if (BR * rd + cb < nv)
        reinterpret_cast<float4*>(Rf + (size_t)(blk0 + BR * rd + cb) * B * B)[rem] =
            *reinterpret_cast<const float4*>(F + (cb * B + rem / (B / 4)) * FP + 4 * (rem % (B / 4)));
    }
  }
  if (Rops == nullptr) return;
  uint32_t pk[RPL][B / 2];
#pragma unroll
  for (int t = 0; t < RPL; ++t)
#pragma unroll
    for (int j = 0; j < B; j += 2) pk[t][j / 2] = pack_bf16x2(a[t][j], a[t][j + 1]);
#pragma unroll
  for (int rd = 0; rd < PER / BR; ++rd) {
    const int bb = sub - BR * rd;
    const bool in = bb >= 0 && bb < BR;
    __syncthreads();
    // R rows in; then R^T rows (columns of R) beside them
    if (in) {
#pragma unroll
      for (int t = 0; t < RPL; ++t)
#pragma unroll
        for (int v = 0; v < B / 8; ++v)
          *reinterpret_cast<uint4*>(O + ((bb * 2) * B + qd + LPB * t) * OP + 8 * v) =
              make_uint4(pk[t][4 * v], pk[t][4 * v + 1], pk[t][4 * v + 2], pk[t][4 * v + 3]);
    }
    __syncthreads();
    if (in) {
      const uint16_t* Rb = O + (bb * 2) * B * OP;
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const int r = qd + LPB * t;
        uint32_t pt[B / 2];
#pragma unroll
        for (int j = 0; j < B; j += 2) pt[j / 2] = (uint32_t)Rb[j * OP + r] | ((uint32_t)Rb[(j + 1) * OP + r] << 16);
#pragma unroll
        for (int v = 0; v < B / 8; ++v)
          *reinterpret_cast<uint4*>(O + ((bb * 2 + 1) * B + r) * OP + 8 * v) =
              make_uint4(pt[4 * v], pt[4 * v + 1], pt[4 * v + 2], pt[4 * v + 3]);
      }
    }
    __syncthreads();
    // a block's pack is 2 B B bf16 = B B / 4 pieces of 16 bytes
#pragma unroll 2
    for (int i = 0; i < BR * B * B / 4 / 64; ++i) {
      const int c = lane + 64 * i, cb = c / (B * B / 4), rem = c % (B * B / 4);
      const int m = rem / (B * B / 8), row = (rem % (B * B / 8)) / (B / 8), c16 = rem % (B / 8);
      if (BR * rd + cb < nv)
        reinterpret_cast<uint4*>(Rops + (size_t)(blk0 + BR * rd + cb) * 2 * B * B)[rem] =
            *reinterpret_cast<const uint4*>(O + ((cb * 2 + m) * B + row) * OP + 8 * c16);
    }
  }
}

// The same solve with two lanes per row (lane 2r + h holds columns
// [16h, 16h + 16) of row r): half the pivot-row reads and half the updates
// per lane on the serial chain of pivot steps, for builds of few blocks,
// where that chain is the whole cost.  PER = 32 / B blocks per wave.  The
// pivots are taken two at a time (a 2 x 2 block K = {s, s + 1}): the
// in-place inversion by block pivots, P = A[K][K],
//   A[i][j] -= A[i][K] P^-1 A[K][j],  A[i][K] = -A[i][K] P^-1   (i, j not in K)
//   A[K][j] = P^-1 A[K][j],           A[K][K] = P^-1,
// equals the two single pivots one after the other (and needs no row
// exchange for the same reason: every principal block of I - Q, Q skew,
// has a positive definite symmetric part), with b / 2 broadcasts through
// LDS on the serial chain instead of b.
template <int B>
__global__ __launch_bounds__(64) void cayley2_kernel(const uint16_t* __restrict__ q, int nblk,
                                                     float* __restrict__ Rf, uint16_t* __restrict__ Rops) {
  constexpr int PER = 32 / B;  // blocks per wave
  constexpr int HB = B / 2;    // columns per lane
  constexpr int NP = B * (B - 1) / 2;
  constexpr int TP = B + 2;  // row pitch (bf16) of the transpose tile
  constexpr int STAGE = PER * NP * 4 > PER * B * TP * 2 ? PER * NP * 4 : PER * B * TP * 2;
  __shared__ __attribute__((aligned(16))) uint8_t stage[STAGE];
  __shared__ __attribute__((aligned(16))) float prow[PER][2][B];  // the two pivot rows

  const int lane = threadIdx.x;
  const int sub = lane / (2 * B), r = (lane / 2) % B, h = lane & 1;
  const int c0 = h * HB;  // first column of this lane
  const int blk0 = blockIdx.x * PER;
  const int nv = min(PER, nblk - blk0);
  const int blk = blk0 + sub;

  // parameters of the wave's blocks (PER * NP contiguous bf16), staged as fp32
  float* qs = reinterpret_cast<float*>(stage);
  const uint16_t* qw = q + (size_t)blk0 * NP;
  const int nq = nv * NP;
  {
    constexpr int NV = (PER * NP + 63) / 64;
    uint16_t v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = qw[min(lane + 64 * k, nq - 1)];  // clamped: no branch
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (lane + 64 * k < nq) qs[lane + 64 * k] = bf16_to_f32(v[k]);
  }
  __syncthreads();

  // A[r][c] = delta_rc - Q[r][c] for this lane's columns
  float a[HB];
  const float* qb = qs + sub * NP;
#pragma unroll
  for (int cc = 0; cc < HB; ++cc) {
    const int c = c0 + cc;
    const int lo = c < r ? c : r, hi = c < r ? r : c;
    const float v = (c == r || sub >= nv) ? 0.0f : qb[lo * B - lo * (lo + 1) / 2 + (hi - lo - 1)];
    a[cc] = c == r ? 1.0f : (c > r ? -v : v);
  }
  __syncthreads();  // stage is reused for the transpose at the end

  auto step = [&](auto tc) {
    constexpr int s = 2 * decltype(tc)::value;  // pivot columns s, s + 1
    constexpr int hs = s / HB, js = s % HB;     // both in lane half hs (HB is even)
    if (r == s || r == s + 1) {
#pragma unroll
      for (int j = 0; j < HB; j += 4)
        *reinterpret_cast<float4*>(&prow[sub][r - s][c0 + j]) = make_float4(a[j], a[j + 1], a[j + 2], a[j + 3]);
    }
    // A[r][K]: held by the lane of half hs of this row
    const float m0 = a[js], m1 = a[js + 1];
    const float o0 = __shfl_xor(m0, 1), o1 = __shfl_xor(m1, 1);
    const float f0 = h == hs ? m0 : o0, f1 = h == hs ? m1 : o1;
    wave_sync();
    float p0[HB], p1[HB];
#pragma unroll
    for (int j = 0; j < HB; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&prow[sub][0][c0 + j]);
      const float4 w = *reinterpret_cast<const float4*>(&prow[sub][1][c0 + j]);
      p0[j] = v.x;
      p0[j + 1] = v.y;
      p0[j + 2] = v.z;
      p0[j + 3] = v.w;
      p1[j] = w.x;
      p1[j + 1] = w.y;
      p1[j + 2] = w.z;
      p1[j + 3] = w.w;
    }
    const float q00 = prow[sub][0][s], q01 = prow[sub][0][s + 1];
    const float q10 = prow[sub][1][s], q11 = prow[sub][1][s + 1];
    const float det = q00 * q11 - q01 * q10;
    float rd = __builtin_amdgcn_rcpf(det);
    rd = fmaf(rd, fmaf(-det, rd, 1.0f), rd);
    const float i00 = q11 * rd, i01 = -q01 * rd, i10 = -q10 * rd, i11 = q00 * rd;  // P^-1
    // one update for every row: a[j] -= u0 p0[j] + u1 p1[j], with u = A[r][K] P^-1
    // off K, and u = e_k - P^-1[k] on pivot row s + k (whose a[j] is p_k[j])
    const bool k0 = r == s, k1 = r == s + 1;
    float u0 = f0 * i00 + f1 * i10, u1 = f0 * i01 + f1 * i11;
    if (k0) {
      u0 = 1.0f - i00;
      u1 = -i01;
    }
    if (k1) {
      u0 = -i10;
      u1 = 1.0f - i11;
    }
#pragma unroll
    for (int j = 0; j < HB; ++j)
      if (h != hs || (j != js && j != js + 1)) a[j] = fmaf(-u0, p0[j], fmaf(-u1, p1[j], a[j]));
    if (h == hs) {
      a[js] = (k0 ? 1.0f : 0.0f) - u0;
      a[js + 1] = (k1 ? 1.0f : 0.0f) - u1;
    }
    wave_sync();
  };
  for_each_index(step, std::make_integer_sequence<int, B / 2>{});

  // row r of A^-1 (this lane's columns); R = 2 A^-1 - I
#pragma unroll
  for (int j = 0; j < HB; ++j) a[j] = 2.0f * a[j] - (c0 + j == r ? 1.0f : 0.0f);
  if (sub < nv) {
    float4* dst = reinterpret_cast<float4*>(Rf + (size_t)blk * B * B + r * B + c0);
#pragma unroll
    for (int j = 0; j < HB; j += 4) dst[j / 4] = make_float4(a[j], a[j + 1], a[j + 2], a[j + 3]);
  }
  if (Rops == nullptr) return;
  uint32_t pk[HB / 2];
#pragma unroll
  for (int j = 0; j < HB; j += 2) pk[j / 2] = pack_bf16x2(a[j], a[j + 1]);
  uint16_t* tt = reinterpret_cast<uint16_t*>(stage) + sub * B * TP;
#pragma unroll
  for (int j = 0; j < HB; j += 2) *reinterpret_cast<uint32_t*>(tt + r * TP + c0 + j) = pk[j / 2];
  __syncthreads();
  uint32_t pt[HB / 2];  // row r of R^T, columns c0 ..: R[c0 + j][r]
#pragma unroll
  for (int j = 0; j < HB; j += 2)
    pt[j / 2] = (uint32_t)tt[(c0 + j) * TP + r] | ((uint32_t)tt[(c0 + j + 1) * TP + r] << 16);
  if (sub < nv) {
    uint4* r0 = reinterpret_cast<uint4*>(Rops + (size_t)blk * 2 * B * B + r * B + c0);          // R, row r
    uint4* r1 = reinterpret_cast<uint4*>(Rops + (size_t)blk * 2 * B * B + B * B + r * B + c0);  // R^T, row r
#pragma unroll
    for (int v = 0; v < HB / 8; ++v) {
      r0[v] = make_uint4(pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]);
      r1[v] = make_uint4(pt[4 * v], pt[4 * v + 1], pt[4 * v + 2], pt[4 * v + 3]);
    }
  }
}

// ---- dequant hook: exactly the bf16 values the matrix cores consume -------
template <int WF>  // a 4-bit format
__global__ __launch_bounds__(256) void dequant_w4_kernel(const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales,
                                                         uint4* __restrict__ out, size_t n8,
                                                         int cols, int g) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n8) return;
  const int per_row = cols / 8;
  const size_t r = idx / per_row;
  const int c = (int)(idx % per_row) * 8;
  out[idx] = W4<WF>::dq(codes[idx], W4<WF>::scale(scales[r * (size_t)(cols / g) + c / g]));
}

__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint2* __restrict__ codes,
                                                          uint4* __restrict__ out, size_t n8) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n8) return;
  const uint2 w = codes[idx];
  const uint2 lo = dq_fp8x4(w.x), hi = dq_fp8x4(w.y);
  out[idx] = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Row-major 4-bit weights to the tiled storage of oft_formats.h, `count`
// [rows, cols] matrices one after another: one thread per 16-byte piece of
// codes (32 columns of a row, which stay together in one tile row), then one
// per scale slot.  A permutation: every byte is copied once.
__global__ __launch_bounds__(256) void pack_t4_codes_kernel(const uint4* __restrict__ codes,
                                                            uint8_t* __restrict__ out, size_t n16, int rows,
                                                            int cols) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n16) return;
  const int per_row = cols / 32;
  const size_t per_mat = (size_t)rows * per_row;
  const size_t m = idx / per_mat, rem = idx % per_mat;
  const int r = (int)(rem / per_row), c = (int)(rem % per_row);
  *reinterpret_cast<uint4*>(out + m * per_mat * 16 + t4_code_off(r, 16 * c, cols)) = codes[idx];
}

__global__ __launch_bounds__(256) void pack_t4_scales_kernel(const uint16_t* __restrict__ scales,
                                                             uint8_t* __restrict__ out, size_t n, int rows,
                                                             int cols, int g) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int per_row = cols / g;
  const size_t per_mat = (size_t)rows * per_row;
  const size_t m = idx / per_mat, rem = idx % per_mat;
  const int r = (int)(rem / per_row), j = (int)(rem % per_row);
  *reinterpret_cast<uint16_t*>(out + m * per_mat * 2 + t4_scale_off(r, j, cols, g)) = scales[idx];
}

hipError_t launch_pack_t4(int count, int rows, int cols, int g, const uint8_t* codes, const uint16_t* scales,
                          uint8_t* codes_t, uint16_t* scales_t, hipStream_t st) {
  const size_t n16 = (size_t)count * rows * (cols / 32);
  const size_t ns = (size_t)count * rows * (cols / g);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_t4_codes_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(codes), codes_t, n16, rows, cols);
  hipLaunchKernelGGL(pack_t4_scales_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st, scales,
                     reinterpret_cast<uint8_t*>(scales_t), ns, rows, cols, g);
  return hipGetLastError();
}

hipError_t launch_cayley(const uint16_t* q, int nblk, int b, float* Rf, uint16_t* Rops,
                         hipStream_t st) {
  if (nblk == 0) return hipSuccess;
  ProfScope prof(st, "cayley");
  // few blocks (at most a few per SIMD): the serial pivot chain is the cost,
  // so two lanes per row; many blocks: throughput, one lane per row
  const bool two = nblk <= 4 * num_cus() * (b == 32 ? 1 : 2);
  if (b == 32 && two)
    hipLaunchKernelGGL(cayley2_kernel<32>, dim3(nblk), dim3(64), 0, st, q, nblk, Rf, Rops);
  else if (b == 32)
    hipLaunchKernelGGL(cayley_kernel<32>, dim3((nblk + 3) / 4), dim3(64), 0, st, q, nblk, Rf, Rops);
  else if (two)
    hipLaunchKernelGGL(cayley2_kernel<16>, dim3((nblk + 1) / 2), dim3(64), 0, st, q, nblk, Rf, Rops);
  else
    hipLaunchKernelGGL(cayley_kernel<16>, dim3((nblk + 3) / 4), dim3(64), 0, st, q, nblk, Rf, Rops);
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int rows, int cols, int g, const uint8_t* codes,
                          const void* scales, uint16_t* out, hipStream_t st) {
  const size_t n8 = (size_t)rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n8 + 255) / 256);
  if (wf_4bit(fmt)) {
    hipLaunchKernelGGL(fmt == WF_FP4 ? dequant_w4_kernel<WF_FP4> : dequant_w4_kernel<WF_INT4>, dim3(grid),
                       dim3(256), 0, st, reinterpret_cast<const uint32_t*>(codes),
                       static_cast<const uint16_t*>(scales), reinterpret_cast<uint4*>(out), n8, cols, g);
  } else {
    hipLaunchKernelGGL(dequant_fp8_kernel, dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const uint2*>(codes), reinterpret_cast<uint4*>(out), n8);
  }
  return hipGetLastError();
}

}  // namespace oft
