// MoE layer with OFT on the split gate/up projection.
//
// Orbit pages: the Synced article, section "Technical details", and the
// chooseai.io release news, section "Dedicated optimisation for low-precision
// MoE models": the router-selected experts are grouped dynamically into
// fixed-size batches, dequantised only temporarily and run as a grouped GEMM,
// so the transient high-precision weight memory stays bounded.  Here the
// dequantised weight never leaves LDS (zero transient weight memory); the
// chunk table of active experts orders the grouped work list.
//
// Routing (all on the device, no host synchronisation):
//   topk    : one wave per token; k rounds of a wave arg-max over the fp32
//             logits (larger value, then lower expert id), softmax over all E
//             by a butterfly reduction;
//   count   : per 64-token tile, a 64-bit LDS mask per expert marking the
//             tile's tokens that selected it (integer OR, order-free);
//   scan    : counts = popcounts summed over tiles, exclusive scans over
//             experts and over tiles by wavefront scans, active list, chunk
//             table, grouped-GEMM work list;
//   permute : rank of a token inside its tile and expert = popcount of the
//             mask bits below its lane, so positions are stable (expert, then
//             token).
#include <utility>

#include "gemm_nn.h"
#include "gemm_nn_dma.h"
#include "gemm_nn_q4.h"
#include "gemm_nt_hl.h"
#include "gemm_nt.h"
#include "gemm_nt_dma.h"
#include "oft_moe.h"
#include "oft_prof.h"

namespace oft {
namespace {

constexpr int MOE_BM = 128;  // rows (expert positions) per grouped tile
constexpr int MOE_NBUF = 1;  // LDS buffers of the grouped GEMMs

// ---------------------------------------------------------------- wave scans
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// exclusive scan of v over the workgroup (blockDim.x a multiple of 64, at
// most 1024): wavefront inclusive scans, then a scan of the wave totals by
// wave 0; also returns the total.  sh needs 33 ints.
__device__ int block_excl_scan(int v, int* total, int* sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int wt = lane < nw ? sh[lane] : 0;
    const int ws = wave_incl_scan(wt);
    if (lane < 16) sh[16 + lane] = ws - wt;
    if (lane == 15) sh[32] = ws;
  }
  __syncthreads();
  const int r = sh[16 + w] + inc - v;
  *total = sh[32];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- top-k
// L lanes per token (64 / L tokens per wave), NV logits per lane (L NV >= E).
// Slot j: the largest logit not yet taken, ties to the lower expert id (NaN
// ranks as -inf, so every slot finds a candidate); lane j of the group keeps
// slot j.
template <int L, int NV>
__global__ __launch_bounds__(256) void moe_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                       int k, int renorm, int* __restrict__ idx,
                                                       float* __restrict__ wout) {
  static_assert(L == 16 || L == 32 || L == 64, "lanes per token");
  static_assert(NV <= 32, "taken mask");
  constexpr int TPW = 64 / L;
  const int lane = threadIdx.x & 63, sl = lane % L;
  const int t = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW + lane / L;
  if (t >= T) return;  // whole groups leave together: the shuffles below stay within a group
  const float* row = logits + (size_t)t * E;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = sl + L * i;
    const float x = e < E ? row[e] : -INFINITY;
    v[i] = x != x ? -INFINITY : x;
  }
  uint32_t taken = 0;
  float mx = 0.0f, myv = 0.0f;
  int mye = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = sl + L * i;
      if (e < E && !((taken >> i) & 1u)) {
        if (v[i] > bv || (v[i] == bv && e < be)) {
          bv = v[i];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be % L == sl) taken |= 1u << (be / L);
    if (sl == j) {
      myv = bv;
      mye = be;
    }
    if (j == 0) mx = bv;
  }
  float s = 0.0f, sel = sl < k ? __expf(myv - mx) : 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (sl + L * i < E) s += __expf(v[i] - mx);
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) {
    s += __shfl_xor(s, off);
    sel += __shfl_xor(sel, off);
  }
  const float den = renorm ? sel : s;
  if (sl < k) {
    idx[(size_t)t * k + sl] = mye;
    wout[(size_t)t * k + sl] = __expf(myv - mx) / den;
  }
}

// Router backward: d_logits[t, e] from dw[t, j], the gradient of the combine
// weights, through the softmax and the fixed top-k selection idx[t, j].
// Without renormalisation dl_e = p_e (g_e - S) for every expert (p the
// softmax of the row, g_e = dw_j where idx_j = e, else 0, S = sum_j dw_j
// w_j); renormalised, w is the softmax of the selected logits alone, so
// dl_{idx_m} = w_m (dw_m - S) and the other experts get 0.  p and w are
// recomputed from the logits with the arithmetic of moe_topk_kernel (a NaN
// logit ranks as -inf there and gets no gradient here).
// L lanes per token (a power of two, 16 .. 64; 64 / L tokens per wave), NV
// logits per lane (L * NV >= E)
template <int L, int NV>
__global__ __launch_bounds__(256) void moe_router_bwd_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                             int renorm, const int* __restrict__ idx,
                                                             const float* __restrict__ dw,
                                                             float* __restrict__ dl) {
  static_assert(L == 16 || L == 32 || L == 64, "lanes per token");
  constexpr int TPW = 64 / L;
  const int lane = threadIdx.x & 63, sl = lane % L;  // lane within the token's group
  const int t = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW + lane / L;
  if (t >= T) return;  // whole groups leave together: the shuffles below stay within a group
  const int g0 = lane - sl;  // first lane of the group
  const float* row = logits + (size_t)t * E;
  // one round trip: the row, the selection and its dw are all in flight
  // before the first is used; the selected logits are read from the row's
  // registers, not loaded again
  int ej = -1;
  float dj = 0.0f;
  if (sl < k) {
    ej = idx[(size_t)t * k + sl];
    dj = dw[(size_t)t * k + sl];
  }
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = sl + L * i;
    const float x = e < E ? row[e] : -INFINITY;
    v[i] = x != x ? -INFINITY : x;
  }
  float mx = v[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) mx = fmaxf(mx, v[i]);
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float p[NV], s = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    p[i] = sl + L * i < E ? __expf(v[i] - mx) : 0.0f;
    s += p[i];
  }
  // dw of the selected experts this lane owns (0 elsewhere); an index
  // outside [0, E) matches no expert
  float g[NV];
  bool in[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    g[i] = 0.0f;
    in[i] = false;
  }
  for (int m = 0; m < k; ++m) {
    const int em = __shfl(ej, g0 + m);
    const float dm = __shfl(dj, g0 + m);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (em == sl + L * i) {
        g[i] = dm;
        in[i] = true;
      }
  }
  // selected mass and sum_j dw_j p_j, reduced together with the row sum
  float sel = 0.0f, gp = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    sel += in[i] ? p[i] : 0.0f;
    gp = fmaf(g[i], p[i], gp);
  }
#pragma unroll
  for (int off = L / 2; off >= 1; off >>= 1) {
    s += __shfl_xor(s, off);
    sel += __shfl_xor(sel, off);
    gp += __shfl_xor(gp, off);
  }
  // w = p / den over the experts that carry weight; S = sum_j dw_j w_j
  const float den = renorm ? sel : s;
  const float S = gp / den;
  float* out = dl + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = sl + L * i;
    if (e < E) {
      const float q = (renorm && !in[i]) ? 0.0f : p[i] / den;
      out[e] = q * (g[i] - S);
    }
  }
}

// ---------------------------------------------------------------- count
__global__ __launch_bounds__(64) void moe_count_kernel(const int* __restrict__ idx, int T, int E, int k,
                                                       unsigned long long* __restrict__ gmask) {
  extern __shared__ unsigned long long smask[];
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  for (int e = lane; e < E; e += 64) smask[e] = 0ull;
  __syncthreads();
  const int t = tile * 64 + lane;
  if (t < T) {
    for (int j = 0; j < k; ++j) atomicOr(&smask[idx[(size_t)t * k + j]], 1ull << lane);
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) gmask[(size_t)tile * E + e] = smask[e];
}

// ---------------------------------------------------------------- scan
__device__ void write_work_list(int cnt_e, int e, int E, int bm, int* list, int* ntiles, int* sh) {
  const int nt_e = e < E ? (cnt_e + bm - 1) / bm : 0;
  int total;
  const int start = block_excl_scan(nt_e, &total, sh);
  for (int i = 0; i < nt_e; ++i) {
    list[2 * (start + i)] = e;
    list[2 * (start + i) + 1] = i * bm;
  }
  if (threadIdx.x == 0) *ntiles = total;
}

// per expert (one workgroup each): counts over the 64-token tiles and the
// exclusive scan over tiles, relative to the expert's first position
__global__ __launch_bounds__(256) void moe_tilescan_kernel(const unsigned long long* __restrict__ gmask,
                                                           int ntile64, int E, int* __restrict__ tile_rel,
                                                           int* __restrict__ counts) {
  __shared__ int sh[40];
  const int e = blockIdx.x;
  int carry = 0;
  for (int t0 = 0; t0 < ntile64; t0 += 256) {
    const int t = t0 + threadIdx.x;
    const int c = t < ntile64 ? __popcll(gmask[(size_t)t * E + e]) : 0;
    int tot;
    const int ex = block_excl_scan(c, &tot, sh);
    if (t < ntile64) tile_rel[(size_t)t * E + e] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// one workgroup: offsets (scan over experts), active list, chunk table and
// the grouped-GEMM work list
__global__ __launch_bounds__(1024) void moe_scan_kernel(int E, int chunk, MoeRoutingDev rt,
                                                        int* __restrict__ list, int* __restrict__ ntiles) {
  __shared__ int sh[40];
  const int e = threadIdx.x;
  const int cnt = e < E ? rt.counts[e] : 0;
  int total;
  const int off = block_excl_scan(cnt, &total, sh);
  if (e < E) rt.offsets[e] = off;
  if (e == 0) rt.offsets[E] = total;
  int nact;
  const int rank = block_excl_scan((e < E && cnt > 0) ? 1 : 0, &nact, sh);
  if (e < E) {
    rt.chunk_of_expert[e] = cnt > 0 ? rank / chunk : -1;
    if (cnt > 0) rt.active[rank] = e;
    if (e >= nact) rt.active[e] = -1;
  }
  if (e == 0) *rt.n_active = nact;
  write_work_list(e < E ? cnt : 0, e, E, MOE_BM, list, ntiles, sh);
}

__global__ __launch_bounds__(1024) void moe_worklist_kernel(const int* __restrict__ counts, int E, int bm,
                                                            int* __restrict__ list, int* __restrict__ ntiles) {
  __shared__ int sh[40];
  const int e = threadIdx.x;
  write_work_list(e < E ? counts[e] : 0, e, E, bm, list, ntiles, sh);
}

// ---------------------------------------------------------------- permute
__global__ __launch_bounds__(64) void moe_permute_kernel(const int* __restrict__ idx, int T, int E, int k,
                                                         const unsigned long long* __restrict__ gmask,
                                                         const int* __restrict__ tile_rel,
                                                         const int* __restrict__ offsets,
                                                         int* __restrict__ perm, int* __restrict__ inv_perm) {
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int t = tile * 64 + lane;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)t * k + j];
    const int rank = __popcll(gmask[(size_t)tile * E + e] & below);
    const int pos = offsets[e] + tile_rel[(size_t)tile * E + e] + rank;
    perm[pos] = t * k + j;
    inv_perm[t * k + j] = pos;
  }
}

// ---------------------------------------------------------------- combine
// y[t] = sum_j w[t, j] * O[inv_perm[t*k + j]], fixed order over j
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ O, int H, int k,
                                                          const int* __restrict__ inv_perm,
                                                          const float* __restrict__ w, size_t n8,
                                                          uint16_t* __restrict__ y) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int per = H / 8;
  const size_t t = i / per;
  const int c = (int)(i % per) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const uint4 v = *reinterpret_cast<const uint4*>(O + (size_t)inv_perm[t * k + j] * H + c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += wj * bf16_to_f32((uint16_t)(u[q >> 1] >> (16 * (q & 1))));
  }
  *reinterpret_cast<uint4*>(y + t * H + c) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                        pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

// dX[t] = sum_j dXp[inv_perm[t*k + j]], fixed order over j
__global__ __launch_bounds__(256) void moe_unpermute_sum_kernel(const uint16_t* __restrict__ dXp, int H, int k,
                                                                const int* __restrict__ inv_perm, size_t n8,
                                                                uint16_t* __restrict__ dx) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int per = H / 8;
  const size_t t = i / per;
  const int c = (int)(i % per) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < k; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(dXp + (size_t)inv_perm[t * k + j] * H + c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += bf16_to_f32((uint16_t)(u[q >> 1] >> (16 * (q & 1))));
  }
  *reinterpret_cast<uint4*>(dx + t * H + c) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

// dw[p] = sum over k tiles of dw_part[kt][inv_perm[p]], fixed order
__global__ __launch_bounds__(256) void moe_dw_reduce_kernel(const float* __restrict__ part, int nkt, long P,
                                                            const int* __restrict__ inv_perm, float* __restrict__ dw) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p >= P) return;
  const int pos = inv_perm[p];
  float s = 0.0f;
  for (int kt = 0; kt < nkt; ++kt) s += part[(size_t)kt * P + pos];
  dw[p] = s;
}

// ---------------------------------------------------------------- dq per expert
// One workgroup per (64 gate/up channels, expert): S = dH_blk^T H_blk over the
// expert's rows (64-row steps through swizzled LDS transposes, MFMA), then the
// Cayley gradient per block in fp32: Gq = (R^T + I) S (I + R) / 2, dp_il =
// Gq_il - Gq_li (b = 32: the two products on the fp32 matrix cores; b = 16:
// cayley_grad_group).  Inactive experts get zeros (S = 0).  When dz != nullptr
// the same pass writes dz = dH_blk R_j (bf16, MFMA), the rotated operand of
// the gate/up dX GEMM, once per dH tile.
constexpr int LDM = 64 + 8;
// dYT / YT row n keeps the row pair of rows 2 rp, 2 rp + 1 at column 2 rp ^
// msw(n): the eight-channel group of n (bits 3..5) XORs the 8-column chunk,
// so the 4-byte transposed stores of a wave (channels 8 c + q, pairs rp)
// fall on 64 different banks and the 16-byte operand reads stay whole chunks.
__device__ __forceinline__ int msw(int n) { return ((n >> 3) & 7) << 3; }

// LDS of one workgroup: the transposed dH / H tiles during the row loop;
// after it, S, then the partial sums of the second wave half (red), whose
// space the Cayley gradient's scratch takes over once S is complete.
template <int B>
struct MoeDqLds {
  static constexpr int TILE = 2 * 64 * LDM * 2;          // dYT + YT
  static constexpr int S_BYTES = 2 * 32 * 33 * 4;         // S[2][32][33]
  static constexpr int RED_BYTES = 2 * 64 * 17 * 4;       // red[2][64][17]
  static constexpr int SCR_BYTES = 3 * (1024 / (B * B)) * B * (B + 4) * 4;
  static constexpr int TAIL = S_BYTES + (RED_BYTES > SCR_BYTES ? RED_BYTES : SCR_BYTES);
  static constexpr int BYTES = TILE > TAIL ? TILE : TAIL;
};

template <int B>
__global__ __launch_bounds__(256) void moe_dq_kernel(const uint16_t* __restrict__ dH, const uint16_t* __restrict__ Hs,
                                                     int ld, const int* __restrict__ offsets,
                                                     const float* __restrict__ Rf, int nblk_e,
                                                     float* __restrict__ dq, const uint16_t* __restrict__ Rops,
                                                     uint16_t* __restrict__ dz) {
  using Lds = MoeDqLds<B>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[Lds::BYTES];
  uint16_t* dYT = reinterpret_cast<uint16_t*>(lds);
  uint16_t* YT = dYT + 64 * LDM;
  auto S = reinterpret_cast<float (*)[32][33]>(lds);
  auto red = reinterpret_cast<float (*)[64][17]>(lds + Lds::S_BYTES);
  // scratch of the Cayley gradient: 3 G B (B + 4) floats, G = 1024 / B^2
  float* scr = reinterpret_cast<float*>(lds + Lds::S_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int n0 = blockIdx.x * 64;
  const int e = blockIdx.y;
  const int m_lo = offsets[e], m_hi = offsets[e + 1];
  const int grp = wave & 1, kh = wave >> 1;
  const int c = tid & 7, rp = tid >> 3;

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  const int rg = wave & 1, rh = wave >> 1;
  const int nbr = n0 + 32 * rg;
  uint4 rtf[2] = {zero4(), zero4()};
  if (dz != nullptr) {
    const uint16_t* re = Rops + (size_t)e * nblk_e * 2 * B * B;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (B == 32) {
        rtf[t] = *reinterpret_cast<const uint4*>(re + (size_t)(nbr / 32) * 2048 + 1024 + l32 * 32 + 16 * t + 8 * g2);
      } else {
        if ((l32 >> 4) == t)
          rtf[t] = *reinterpret_cast<const uint4*>(re + (size_t)(nbr / 16 + t) * 512 + 256 + (l32 & 15) * 16 + 8 * g2);
      }
    }
  }
  // registers one 64-row step ahead: the dz operand rows (f) and the dH / H
  // rows of the cross product (d, y)
  uint4 f[2], d[2], y[2];
  auto load = [&](int ms) {
    if (dz != nullptr) {
      const int m = ms + 32 * rh + l32;
      const bool mok = m < m_hi;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        f[t] = mok ? *reinterpret_cast<const uint4*>(dH + (size_t)m * ld + nbr + 16 * t + 8 * g2) : zero4();
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = ms + 2 * rp + h;
      const bool ok = m < m_hi;
      d[h] = ok ? *reinterpret_cast<const uint4*>(dH + (size_t)m * ld + n0 + 8 * c) : zero4();
      y[h] = ok ? *reinterpret_cast<const uint4*>(Hs + (size_t)m * ld + n0 + 8 * c) : zero4();
    }
  };
  if (m_lo < m_hi) load(m_lo);
  for (int ms = m_lo; ms < m_hi; ms += 64) {
    if (dz != nullptr) {
      const int m = ms + 32 * rh + l32;
      const bool mok = m < m_hi;
      f32x16 o;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = 0.0f;
      o = mfma32(as_bf16x8(rtf[0]), as_bf16x8(f[0]), o);
      o = mfma32(as_bf16x8(rtf[1]), as_bf16x8(f[1]), o);
      // lane (l32, g2) holds channels 8 q + 4 g2 + [0, 4) of row m; the two
      // halves of the wave exchange (v_permlane32_swap: lanes 32..63 of the
      // first operand with lanes 0..31 of the second) so that lane g2 = 0
      // holds channels 8 q + [0, 8) for q = 0, 2 and lane g2 = 1 for q = 1,
      // 3: two 16-byte stores per lane, 32 contiguous bytes per row each
      uint32_t pk[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pk[q][0] = pack_bf16x2(o[4 * q], o[4 * q + 1]);
        pk[q][1] = pack_bf16x2(o[4 * q + 2], o[4 * q + 3]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t lo[2], hi[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const auto sw = __builtin_amdgcn_permlane32_swap(pk[2 * h][w], pk[2 * h + 1][w], false, false);
          lo[w] = sw[0];
          hi[w] = sw[1];
        }
        if (mok)
          *reinterpret_cast<uint4*>(dz + (size_t)m * ld + nbr + 8 * (2 * h + g2)) = make_uint4(lo[0], lo[1], hi[0], hi[1]);
      }
    }
    __syncthreads();
    {
      const uint32_t d0[4] = {d[0].x, d[0].y, d[0].z, d[0].w}, d1[4] = {d[1].x, d[1].y, d[1].z, d[1].w};
      const uint32_t y0[4] = {y[0].x, y[0].y, y[0].z, y[0].w}, y1[4] = {y[1].x, y[1].y, y[1].z, y[1].w};
      if (ms + 64 < m_hi) load(ms + 64);  // in flight during the transposes and MFMAs below
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
        const int n = 8 * c + q;
        *reinterpret_cast<uint32_t*>(&dYT[n * LDM + ((2 * rp) ^ msw(n))]) =
            __builtin_amdgcn_perm(d1[q >> 1], d0[q >> 1], sel);
        *reinterpret_cast<uint32_t*>(&YT[n * LDM + ((2 * rp) ^ msw(n))]) =
            __builtin_amdgcn_perm(y1[q >> 1], y0[q >> 1], sel);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const int kk = 2 * kh + kq;
      const int n = 32 * grp + l32;
      const int mo = (16 * kk + 8 * g2) ^ msw(n);
      acc = mfma32(*reinterpret_cast<const bf16x8*>(&dYT[n * LDM + mo]),
                   *reinterpret_cast<const bf16x8*>(&YT[n * LDM + mo]), acc);
    }
  }
  if (dq == nullptr) return;
  __syncthreads();  // the transposed tiles are dead: their space holds S and red
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[grp][lane][r] = acc[r];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[grp][(r / 4) * 8 + 4 * g2 + (r % 4)][l32] = acc[r] + red[grp][lane][r];
  }
  __syncthreads();
  constexpr int GB = 1024 / (B * B), NP = B * (B - 1) / 2;
  if constexpr (B == 32) {
    // the two blocks' gradients on the fp32 matrix cores, wave w < 2 taking
    // block w: T1 = S + S R (D = A B + C with A = S, B = R, C = S), then
    // 2 Gq = T1 + R^T T1 (A = R^T, B = T1, C = T1); in step s of
    // v_mfma_f32_32x32x2f32 lane (l32, g2) supplies A[l32][2 s + g2] and
    // B[2 s + g2][l32], and holds D[8 (r / 4) + 4 g2 + r % 4][l32] in r
    auto T1 = reinterpret_cast<float (*)[32][33]>(lds + Lds::S_BYTES);  // the dead partial sums' space
    const int bk = wave;
    const int jb0 = n0 / 32 + bk;
    if (wave < 2 && jb0 < nblk_e) {
      const float* Rg = Rf + ((size_t)e * nblk_e + jb0) * 1024;
      float rk[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) rk[s2] = Rg[(2 * s2 + g2) * 32 + l32];
      f32x16 t;
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = S[bk][(r / 4) * 8 + 4 * g2 + (r % 4)][l32];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) t = __builtin_amdgcn_mfma_f32_32x32x2f32(S[bk][l32][2 * s2 + g2], rk[s2], t, 0, 0, 0);
      // (LDS accesses of one wave complete in order: T1 is read back below,
      // S is overwritten after its last read)
#pragma unroll
      for (int r = 0; r < 16; ++r) T1[bk][(r / 4) * 8 + 4 * g2 + (r % 4)][l32] = t[r];
      f32x16 g = t;
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) g = __builtin_amdgcn_mfma_f32_32x32x2f32(rk[s2], T1[bk][2 * s2 + g2][l32], g, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) S[bk][(r / 4) * 8 + 4 * g2 + (r % 4)][l32] = 0.5f * g[r];
    }
    __syncthreads();
    // dp_il = Gq_il - Gq_li, row-major upper triangle of each block: thread
    // (block tid / 128, row i, columns 8 (tid % 4) .. + 7 above the
    // diagonal), packed index i B - i (i + 1) / 2 + l - i - 1
    const int b2 = tid >> 7, i = (tid & 127) >> 2, c8 = 8 * (tid & 3);
    if (n0 / 32 + b2 < nblk_e) {
      float* dst = dq + ((size_t)e * nblk_e + n0 / 32 + b2) * NP + (i * 32 - i * (i + 1) / 2 - i - 1);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int l = c8 + k;
        if (l > i) dst[l] = S[b2][i][l] - S[b2][l][i];
      }
    }
    return;
  }
  // the blocks of the 64 channels, G at a time
#pragma unroll
  for (int q = 0; q < 64 / (GB * B); ++q) {
    const int j0 = n0 / B + q * GB;  // first block (within the expert) of the group
    if (j0 >= nblk_e) break;         // uniform
    const size_t jb = (size_t)e * nblk_e + j0;
    cayley_grad_group<B>(scr, Rf + jb * B * B, dq + jb * NP, min(GB, nblk_e - j0), tid, [&](int g, int r, int cc) {
      const int ch = (q * GB + g) * B;  // first channel of the block in the 64
      const float* row = &S[ch / 32][ch % 32 + r][ch % 32 + cc];
      return make_float4(row[0], row[1], row[2], row[3]);
    });
    __syncthreads();
  }
}

hipError_t last() { return hipGetLastError(); }

}  // namespace

MoeWs moe_ws_layout(const MoeDims& d, int pass) {
  MoeWs w{};
  const long P = (long)d.T * d.k;
  const int nt64 = (d.T + 63) / 64;
  const long max_tiles = (P + MOE_BM - 1) / MOE_BM + d.E;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.list = take(2 * max_tiles * sizeof(int));
  w.ntiles = take(sizeof(int));
  w.max_tiles = max_tiles;
  if (pass == 0) {
    w.max_tiles64 = (P + 15) / 16 + d.E;  // tiles of 16 or 64 rows
    w.list64 = take(2 * w.max_tiles64 * sizeof(int));
    w.ntiles64 = take(sizeof(int));
    w.gmask = take((size_t)nt64 * d.E * 8);
    w.tile_off = take((size_t)nt64 * d.E * 4);
    w.act = take((size_t)P * d.I * 2);
    w.O = take((size_t)P * d.H * 2);
  } else {
    w.dH = take((size_t)P * 2 * d.I * 2);
    w.dw_part = take((size_t)((d.I + 127) / 128) * P * 4);
    w.dXp = take((size_t)P * d.H * 2);
    w.dz = take((size_t)P * 2 * d.I * 2);
  }
  w.bytes = off;
  return w;
}

// Lane-group shape of the per-token router kernels (top-k, router backward):
// f(L, NV) with L lanes per token and NV logits per lane for E experts
// (E <= 1024; L >= 16 >= k, so a token's k slots live on its own group).
template <class F>
static void router_shape(int E, F&& f) {
  using std::integral_constant;
  if (E <= 64)
    f(integral_constant<int, 16>{}, integral_constant<int, 4>{});
  else if (E <= 128)
    f(integral_constant<int, 16>{}, integral_constant<int, 8>{});
  else if (E <= 256)
    f(integral_constant<int, 32>{}, integral_constant<int, 8>{});
  else if (E <= 384)
    f(integral_constant<int, 64>{}, integral_constant<int, 6>{});
  else if (E <= 512)
    f(integral_constant<int, 64>{}, integral_constant<int, 8>{});
  else
    f(integral_constant<int, 64>{}, integral_constant<int, 16>{});
}

hipError_t launch_moe_route(const MoeDims& d, const float* logits, const MoeRoutingDev& rt, char* ws,
                            const MoeWs& L, hipStream_t st) {
  const int nt64 = (d.T + 63) / 64;
  int* list = reinterpret_cast<int*>(ws + L.list);
  int* ntiles = reinterpret_cast<int*>(ws + L.ntiles);
  ProfScope prof(st, "moe.route");
  if (d.T > 0) {
    router_shape(d.E, [&](auto l, auto nv) {
      constexpr int Lc = decltype(l)::value, NVc = decltype(nv)::value;
      const int per = 4 * (64 / Lc);  // tokens per workgroup
      hipLaunchKernelGGL((moe_topk_kernel<Lc, NVc>), dim3((d.T + per - 1) / per), dim3(256), 0, st, logits, d.T,
                         d.E, d.k, d.renorm, rt.topk_idx, rt.topk_w);
    });
    hipLaunchKernelGGL(moe_count_kernel, dim3(nt64), dim3(64), (size_t)d.E * 8, st, rt.topk_idx, d.T, d.E, d.k,
                       reinterpret_cast<unsigned long long*>(ws + L.gmask));
  }
  // (with no tokens the tile loop is empty and every count is written as 0)
  hipLaunchKernelGGL(moe_tilescan_kernel, dim3(d.E), dim3(256), 0, st,
                     reinterpret_cast<const unsigned long long*>(ws + L.gmask), nt64, d.E,
                     reinterpret_cast<int*>(ws + L.tile_off), rt.counts);
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), 0, st, d.E, d.chunk, rt, list, ntiles);
  if (d.T > 0)
    hipLaunchKernelGGL(moe_permute_kernel, dim3(nt64), dim3(64), 0, st, rt.topk_idx, d.T, d.E, d.k,
                       reinterpret_cast<const unsigned long long*>(ws + L.gmask),
                       reinterpret_cast<const int*>(ws + L.tile_off), rt.offsets, rt.perm, rt.inv_perm);
  return last();
}

// W4F: the 4-bit format of the weights when they are not bf16; GEPI: the
// gate/up epilogue, EPI_ROT_SWIGLU (the adapted layer) or EPI_BASE_SWIGLU
// (the frozen base alone: no rotation, h stored only when q.h_saved is set)
template <int B, int W4F, int GEPI>
static hipError_t moe_fwd_gemms(const MoeDims& d, const MoeFwdPtrs& q, const MoeRoutingDev& rt, char* ws,
                                const MoeWs& L, hipStream_t st) {
  const long P = (long)d.T * d.k;
  int* list = reinterpret_cast<int*>(ws + L.list);
  int* ntiles = reinterpret_cast<int*>(ws + L.ntiles);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
  uint16_t* O = reinterpret_cast<uint16_t*>(ws + L.O);
  const int nblk_e = 2 * d.I / B;
  // experts averaging at least 64 rows: copy-ring kernels on 128-row tiles;
  // fewer (decode): the weight-streaming copy-ring kernel on 64-row tiles,
  // or on 16-row tiles (deeper weight ring) when they average at most 8
  // (bf16 reference weights: the 128-row copy-ring kernel at every size)
  const bool w16 = d.wf == WF_BF16;
  const bool dma = w16 || (long)d.T * d.k >= 64L * d.E;
  const bool dec = !dma;
  const bool dec16 = dec && (long)d.T * d.k <= 8L * d.E;
  const long wb2 = w16 ? 4 : 1;  // bytes per two weights
  int* list64 = reinterpret_cast<int*>(ws + L.list64);
  int* ntiles64 = reinterpret_cast<int*>(ws + L.ntiles64);
  if (dec) {
    ProfScope prof(st, "moe.worklist");
    hipLaunchKernelGGL(moe_worklist_kernel, dim3(1), dim3(1024), 0, st, rt.counts, d.E, dec16 ? 16 : 64, list64,
                       ntiles64);
  }
  {
    ProfScope prof(st, "moe.gateup");
    NtArgs p{};
    p.a = q.x;
    p.lda = d.H;
    p.wc = q.wgu_codes;
    p.ws = q.wgu_scales;
    p.wc_e = (long)2 * d.I * d.H / 2 * wb2;
    p.ws_e = w16 ? 0 : (long)2 * d.I * (d.H / d.g);
    p.rops = q.R_ops;
    p.rops_e = GEPI == EPI_ROT_SWIGLU ? (long)nblk_e * 2 * B * B : 0;
    p.out = q.h_saved;
    p.ldo = 2 * d.I;
    p.act = act;
    p.ldact = d.I;
    p.M = 0;
    p.K = d.H;
    p.N = 2 * d.I;
    p.g = d.g;
    p.half_n = d.I;
    p.tiles = list;
    p.ntiles = ntiles;
    p.offsets = rt.offsets;
    p.perm = rt.perm;
    p.kslots = d.k;
    if (dma) {
      dim3 grid((d.I + ntd::BN / 2 - 1) / (ntd::BN / 2), (unsigned)L.max_tiles);
      if constexpr (wf_tiled(W4F)) {  // (tiled INT4: H % 256 == 0 and I % 256 == 0)
        hipLaunchKernelGGL((gemm_nt_hl_kernel<W4F, B, GEPI, true>), grid, dim3(nth::NTHR), 0, st, p);
      } else if (w16) {
        hipLaunchKernelGGL((gemm_nt_dma_kernel<WF_BF16, B, MOE_BM, GEPI, false, true>), grid,
                           dim3(ntd::NTHR), 0, st, p);
      } else if (d.H % 128 == 0) {  // weight stages of two K steps (half-line copies)
        hipLaunchKernelGGL((gemm_nt_hl_kernel<W4F, B, GEPI, true>), grid, dim3(nth::NTHR), 0, st, p);
      } else {
        hipLaunchKernelGGL((gemm_nt_dma_kernel<W4F, B, MOE_BM, GEPI, false, true>), grid,
                           dim3(ntd::NTHR), 0, st, p);
      }
    } else {
      p.tiles = list64;
      p.ntiles = ntiles64;
      dim3 grid((d.I + ntd::DEC_BN / 2 - 1) / (ntd::DEC_BN / 2), (unsigned)L.max_tiles64);
      if (d.H % 256 == 0 && dec16) {  // whole-line weight copies on 256-wide steps
        hipLaunchKernelGGL((gemm_nt_dec4_kernel<B, GEPI, true, 16, W4F>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
      } else if (d.H % 256 == 0) {
        hipLaunchKernelGGL((gemm_nt_dec4_kernel<B, GEPI, true, 64, W4F>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
      } else if constexpr (!wf_tiled(W4F)) {
        if (dec16)
          hipLaunchKernelGGL((gemm_nt_dec_kernel<W4F, B, GEPI, true, 16>), grid, dim3(ntd::DEC_NTHR), 0,
                             st, p);
        else
          hipLaunchKernelGGL((gemm_nt_dec_kernel<W4F, B, GEPI, true>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
      }
    }
  }
  {
    ProfScope prof(st, "moe.down");
    NtArgs p{};
    p.a = act;
    p.lda = d.I;
    p.wc = q.wd_codes;
    p.ws = q.wd_scales;
    p.wc_e = (long)d.H * d.I / 2 * wb2;
    p.ws_e = w16 ? 0 : (long)d.H * (d.I / d.g);
    p.rops = q.R_ops;
    p.rops_e = 0;
    p.out = O;
    p.ldo = d.H;
    p.M = 0;
    p.K = d.I;
    p.N = d.H;
    p.g = d.g;
    p.tiles = list;
    p.ntiles = ntiles;
    p.offsets = rt.offsets;
    p.perm = rt.perm;
    p.kslots = 0;
    if (dma) {
      dim3 grid((d.H + ntd::BN - 1) / ntd::BN, (unsigned)L.max_tiles);
      if constexpr (wf_tiled(W4F)) {
        hipLaunchKernelGGL((gemm_nt_hl_kernel<W4F, 32, EPI_PLAIN, true>), grid, dim3(nth::NTHR), 0, st, p);
      } else if (w16) {
        hipLaunchKernelGGL((gemm_nt_dma_kernel<WF_BF16, 32, MOE_BM, EPI_PLAIN, false, true>), grid,
                           dim3(ntd::NTHR), 0, st, p);
      } else if (d.I % 128 == 0) {  // weight stages of two K steps (half-line copies)
        hipLaunchKernelGGL((gemm_nt_hl_kernel<W4F, 32, EPI_PLAIN, true>), grid, dim3(nth::NTHR), 0, st, p);
      } else {
        hipLaunchKernelGGL((gemm_nt_dma_kernel<W4F, 32, MOE_BM, EPI_PLAIN, false, true>), grid,
                           dim3(ntd::NTHR), 0, st, p);
      }
    } else {
      p.tiles = list64;
      p.ntiles = ntiles64;
      dim3 grid((d.H + ntd::DEC_BN - 1) / ntd::DEC_BN, (unsigned)L.max_tiles64);
      if (d.I % 256 == 0 && dec16) {
        hipLaunchKernelGGL((gemm_nt_dec4_kernel<32, EPI_PLAIN, true, 16, W4F>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
      } else if (d.I % 256 == 0) {
        hipLaunchKernelGGL((gemm_nt_dec4_kernel<32, EPI_PLAIN, true, 64, W4F>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
      } else if constexpr (!wf_tiled(W4F)) {
        if (dec16)
          hipLaunchKernelGGL((gemm_nt_dec_kernel<W4F, 32, EPI_PLAIN, true, 16>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
        else
          hipLaunchKernelGGL((gemm_nt_dec_kernel<W4F, 32, EPI_PLAIN, true>), grid, dim3(ntd::DEC_NTHR), 0, st, p);
      }
    }
  }
  const size_t n8 = (size_t)d.T * d.H / 8;
  if (n8 > 0) {
    ProfScope prof(st, "moe.combine");
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, O, d.H, d.k,
                       rt.inv_perm, rt.topk_w, n8, q.y);
  }
  (void)P;
  return last();
}

hipError_t launch_moe_fwd(const MoeDims& d, const float* logits, const MoeFwdPtrs& q, const MoeRoutingDev& rt,
                          char* ws, const MoeWs& L, hipStream_t st, bool base) {
  hipError_t err = launch_moe_route(d, logits, rt, ws, L, st);
  if (err != hipSuccess) return err;
  if (d.T == 0) return hipSuccess;
  if (base)  // the frozen base alone: the block size plays no part
    return d.wf == WF_FP4     ? moe_fwd_gemms<32, WF_FP4, EPI_BASE_SWIGLU>(d, q, rt, ws, L, st)
           : d.wf == WF_INT4T ? moe_fwd_gemms<32, WF_INT4T, EPI_BASE_SWIGLU>(d, q, rt, ws, L, st)
                              : moe_fwd_gemms<32, WF_INT4, EPI_BASE_SWIGLU>(d, q, rt, ws, L, st);
  if (d.wf == WF_FP4)
    return d.b == 32 ? moe_fwd_gemms<32, WF_FP4, EPI_ROT_SWIGLU>(d, q, rt, ws, L, st)
                     : moe_fwd_gemms<16, WF_FP4, EPI_ROT_SWIGLU>(d, q, rt, ws, L, st);
  if (d.wf == WF_INT4T)
    return d.b == 32 ? moe_fwd_gemms<32, WF_INT4T, EPI_ROT_SWIGLU>(d, q, rt, ws, L, st)
                     : moe_fwd_gemms<16, WF_INT4T, EPI_ROT_SWIGLU>(d, q, rt, ws, L, st);
  return d.b == 32 ? moe_fwd_gemms<32, WF_INT4, EPI_ROT_SWIGLU>(d, q, rt, ws, L, st)
                   : moe_fwd_gemms<16, WF_INT4, EPI_ROT_SWIGLU>(d, q, rt, ws, L, st);
}

template <int B, int W4F>
static hipError_t moe_bwd_t(const MoeDims& d, const MoeBwdPtrs& q, const MoeRoutingDev& rt, char* ws,
                            const MoeWs& L, hipStream_t st) {
  const long P = (long)d.T * d.k;
  int* list = reinterpret_cast<int*>(ws + L.list);
  int* ntiles = reinterpret_cast<int*>(ws + L.ntiles);
  uint16_t* dH = reinterpret_cast<uint16_t*>(ws + L.dH);
  float* dw_part = reinterpret_cast<float*>(ws + L.dw_part);
  uint16_t* dXp = reinterpret_cast<uint16_t*>(ws + L.dXp);
  const int nblk_e = 2 * d.I / B;
  const bool w16 = d.wf == WF_BF16;
  const long wb2 = w16 ? 4 : 1;  // bytes per two weights
  {
    ProfScope prof(st, "moe.worklist");
    hipLaunchKernelGGL(moe_worklist_kernel, dim3(1), dim3(1024), 0, st, rt.counts, d.E, MOE_BM, list, ntiles);
  }
  if (d.T > 0) {
    NnArgs p{};
    p.src = q.dy;
    p.lds = d.H;
    p.wc = q.wd_codes;
    p.ws = q.wd_scales;
    p.wc_e = (long)d.H * d.I / 2 * wb2;
    p.ws_e = w16 ? 0 : (long)d.H * (d.I / d.g);
    p.rops = q.R_ops;
    p.out = dH;
    p.ldo = 2 * d.I;
    p.M = 0;
    p.K = d.I;
    p.N = d.H;
    p.g = d.g;
    p.tiles = list;
    p.ntiles = ntiles;
    p.offsets = rt.offsets;
    p.perm = rt.perm;
    p.kslots = d.k;
    p.hsave = q.h_saved;
    p.ldh = 2 * d.I;
    p.topk_w = rt.topk_w;
    p.dw_part = dw_part;
    p.P = P;
    // experts averaging at least 64 rows: the copy-ring NN kernel (faster
    // there; with fewer rows the two-workgroups-per-CU kernel is)
    int nkt;  // column tiles = partial sums of dw per position
    if (wf_tiled(W4F) || (W4F == WF_INT4 && !w16 && d.I % nnq::BKO == 0)) {
      // INT4: codes and scales to LDS by copies, transposed 4-bit operand
      // reads, every code dequantised by one wave
      ProfScope prof(st, "moe.dA");
      dim3 grid(d.I / nnq::BKO, (unsigned)L.max_tiles);
      hipLaunchKernelGGL((gemm_nn_q4_kernel<EPI_SWIGLU_BWD, true, wf_tiled(W4F)>), grid, dim3(nnq::NTHR), 0, st, p);
      nkt = d.I / nnq::BKO;
    } else if constexpr (wf_tiled(W4F)) {
      nkt = 0;  // (not reached: tiled INT4 takes the branch above)
    } else if ((long)d.T * d.k >= 64L * d.E) {
      ProfScope prof(st, "moe.dA");
      dim3 grid((d.I + nnd::BKO - 1) / nnd::BKO, (unsigned)L.max_tiles);
      if (w16)
        hipLaunchKernelGGL((gemm_nn_dma_kernel<WF_BF16, EPI_SWIGLU_BWD, true>), grid, dim3(nnd::NTHR), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_nn_dma_kernel<W4F, EPI_SWIGLU_BWD, true>), grid, dim3(nnd::NTHR), 0, st, p);
      nkt = (d.I + nnd::BKO - 1) / nnd::BKO;
    } else {
      ProfScope prof(st, "moe.dA");
      dim3 grid((d.I + nn::BKO - 1) / nn::BKO, (unsigned)L.max_tiles);
      if (w16)
        hipLaunchKernelGGL((gemm_nn_kernel<MOE_BM, false, WF_BF16, B, PRO_NONE, EPI_SWIGLU_BWD, true, MOE_NBUF>),
                           grid, dim3(256), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_nn_kernel<MOE_BM, false, W4F, B, PRO_NONE, EPI_SWIGLU_BWD, true, MOE_NBUF>),
                           grid, dim3(256), 0, st, p);
      nkt = (d.I + nn::BKO - 1) / nn::BKO;
    }
    if (q.dw) {
      ProfScope prof(st, "moe.dw_reduce");
      hipLaunchKernelGGL(moe_dw_reduce_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, st, dw_part, nkt, P,
                         rt.inv_perm, q.dw);
    }
  }
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + L.dz);
  if (q.dq || (q.dx && d.T > 0)) {
    ProfScope prof(st, "moe.dq");
    hipLaunchKernelGGL(moe_dq_kernel<B>, dim3(2 * d.I / 64, d.E), dim3(256), 0, st, dH, q.h_saved, 2 * d.I,
                       rt.offsets, q.R_f32, nblk_e, q.dq, q.R_ops, (q.dx && d.T > 0) ? dz : nullptr);
  }
  if (q.dx && d.T > 0) {
    {
    ProfScope prof(st, "moe.dX");
    NnArgs p{};
    p.src = dz;
    p.lds = 2 * d.I;
    p.wc = q.wgu_codes;
    p.ws = q.wgu_scales;
    p.wc_e = (long)2 * d.I * d.H / 2 * wb2;
    p.ws_e = w16 ? 0 : (long)2 * d.I * (d.H / d.g);
    p.rops = q.R_ops;
    p.rops_e = (long)nblk_e * 2 * B * B;
    p.out = dXp;
    p.ldo = d.H;
    p.M = 0;
    p.K = d.H;
    p.N = 2 * d.I;
    p.g = d.g;
    p.tiles = list;
    p.ntiles = ntiles;
    p.offsets = rt.offsets;
    p.perm = rt.perm;
    p.kslots = 0;
    if (wf_tiled(W4F) || (W4F == WF_INT4 && !w16 && d.H % nnq::BKO == 0)) {
      dim3 grid(d.H / nnq::BKO, (unsigned)L.max_tiles);
      hipLaunchKernelGGL((gemm_nn_q4_kernel<EPI_STORE, true, wf_tiled(W4F)>), grid, dim3(nnq::NTHR), 0, st, p);
    } else if constexpr (!wf_tiled(W4F)) {
      dim3 grid((d.H + nn::BKO - 1) / nn::BKO, (unsigned)L.max_tiles);
      if (w16)
        hipLaunchKernelGGL((gemm_nn_kernel<MOE_BM, false, WF_BF16, B, PRO_NONE, EPI_STORE, true, MOE_NBUF>), grid,
                           dim3(256), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_nn_kernel<MOE_BM, false, W4F, B, PRO_NONE, EPI_STORE, true, MOE_NBUF>), grid,
                           dim3(256), 0, st, p);
    }
    }
    const size_t n8 = (size_t)d.T * d.H / 8;
    ProfScope prof(st, "moe.unpermute");
    hipLaunchKernelGGL(moe_unpermute_sum_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, dXp, d.H,
                       d.k, rt.inv_perm, n8, q.dx);
  }
  return last();
}

hipError_t launch_moe_bwd(const MoeDims& d, const MoeBwdPtrs& q, const MoeRoutingDev& rt, char* ws,
                          const MoeWs& L, hipStream_t st) {
  if (d.wf == WF_FP4)
    return d.b == 32 ? moe_bwd_t<32, WF_FP4>(d, q, rt, ws, L, st) : moe_bwd_t<16, WF_FP4>(d, q, rt, ws, L, st);
  if (d.wf == WF_INT4T)
    return d.b == 32 ? moe_bwd_t<32, WF_INT4T>(d, q, rt, ws, L, st) : moe_bwd_t<16, WF_INT4T>(d, q, rt, ws, L, st);
  return d.b == 32 ? moe_bwd_t<32, WF_INT4>(d, q, rt, ws, L, st) : moe_bwd_t<16, WF_INT4>(d, q, rt, ws, L, st);
}

hipError_t launch_moe_router_bwd(const MoeDims& d, const float* logits, const int* topk_idx, const float* dw,
                                 float* d_logits, hipStream_t st) {
  if (d.T == 0) return hipSuccess;
  ProfScope prof(st, "moe.router_bwd");
  router_shape(d.E, [&](auto l, auto nv) {
    constexpr int Lc = decltype(l)::value, NVc = decltype(nv)::value;
    const int per = 4 * (64 / Lc);  // tokens per workgroup
    hipLaunchKernelGGL((moe_router_bwd_kernel<Lc, NVc>), dim3((d.T + per - 1) / per), dim3(256), 0, st, logits,
                       d.T, d.E, d.k, d.renorm, topk_idx, dw, d_logits);
  });
  return hipGetLastError();
}

}  // namespace oft
