// Backward of the OFT linear layer.
//
//   dX = rot_R^T(dY) . dequant(W0)        (no gradient of the frozen base:
//                                           the Synced article on Orbit,
//                                           "Technical details", bypasses the
//                                           base-weight gradient GEMM)
//   dQ: S_j = dY_blk^T Y_blk, G_j = S_j R_j (= dY_blk^T Z_blk, Z = Y R),
//       dL/dQ_j = (R_j^T + I) G_j (R_j^T + I) / 2, packed dp_il = Gq_il - Gq_li.
//
// dX = dZ' . W with dZ' = (dY_blk R_j) * s_n (FP8 channel scale): the
// rotation is a prologue of the dX GEMM.  For narrow layers (dX at most two
// 128-column tiles wide) it runs inside gemm_nn_kernel (PRO_ROT); for wider
// layers it would be recomputed once per column tile, so it runs once per dY
// tile inside the dQ pass below (which reads dY anyway) and the dX GEMM
// consumes the rotated bf16 tile.  The dX GEMM contracts over the weight's
// rows, against its storage order; for wide layers with many tokens the
// weight is first rewritten transposed into the workspace (FP8: the codes,
// whose channel scale is already folded into dZ'; INT4: the dequantised bf16
// values, since its group scale varies along the contraction), a pass over
// the weight bytes only, and dX runs on gemm_nt_dma_kernel (gemm_nt_dma.h)
// with a plain epilogue.  Otherwise gemm_nn_kernel reads the weight rows
// directly and transposes tiles through LDS.
// dQ: stage 1 transposes 64 x 64 tiles of dY and Y through LDS and forms the
// b x b cross products S on the matrix cores, one fp32 partial per M slice;
// stage 2 reduces the slices in a fixed order and applies the Cayley
// gradient in fp32 with R_f32.
#include "gemm_nn.h"
#include "gemm_nn_q4.h"
#include "gemm_nt_dma.h"
#include "oft_launch.h"
#include "oft_prof.h"

namespace oft {
namespace {

// ---------------------------------------------------------------- dq stage 1
constexpr int LDM = 64 + 8;

// dYT / YT row n keeps token m at column m ^ msw(n) (16-token groups XORed by
// bits 3..4 of n): the transposed 4-byte stores of a wave hit every bank
// twice at most, 16-byte operand reads stay contiguous.
__device__ __forceinline__ int msw(int n) { return ((n >> 3) & 3) << 4; }

// Besides the partial cross products, when dz != nullptr the kernel writes
// the rotated upstream gradient dz = (dY_blk R_j) * s (s: FP8 channel scale,
// else 1) in bf16: the rotation runs on the matrix cores once per dY tile
// (dZ^T = R_j^T dY^T, accumulator rows are channels), for the dX GEMM.
template <bool YF32, bool FP8, int B>
__global__ __launch_bounds__(256) void dq_partial_kernel(const uint16_t* __restrict__ dy,
                                                         const void* __restrict__ yv,
                                                         float* __restrict__ part, int M, int N,
                                                         int rows_per_split, int ng32,
                                                         const uint16_t* __restrict__ Rops,
                                                         const float* __restrict__ fp8_scale,
                                                         uint16_t* __restrict__ dz) {
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

  // rotation operands of this wave: 32-channel group rg = wave & 1, token
  // half rh = wave >> 1 of each 64-token step
  const int rg = wave & 1, rh = wave >> 1;
  const int nbr = n0 + 32 * rg;
  const bool rot = dz != nullptr && nbr < N;
  uint4 rtf[2] = {zero4(), zero4()};
  float sc[16];
  if (rot) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (B == 32) {
        rtf[t] = *reinterpret_cast<const uint4*>(Rops + (size_t)(nbr / 32) * 2048 + 1024 + l32 * 32 + 16 * t + 8 * g2);
      } else {
        if ((l32 >> 4) == t)
          rtf[t] = *reinterpret_cast<const uint4*>(Rops + (size_t)(nbr / 16 + t) * 512 + 256 + (l32 & 15) * 16 + 8 * g2);
      }
    }
    if constexpr (FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(fp8_scale + nbr + 8 * q + 4 * g2);
        sc[4 * q] = v.x;
        sc[4 * q + 1] = v.y;
        sc[4 * q + 2] = v.z;
        sc[4 * q + 3] = v.w;
      }
    }
  }

  for (int ms = m_lo; ms < m_hi; ms += 64) {
    if (rot) {
      const int m = ms + 32 * rh + l32;
      const bool mok = m < m_hi;
      uint4 f[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        f[t] = mok ? *reinterpret_cast<const uint4*>(dy + (size_t)m * N + nbr + 16 * t + 8 * g2) : zero4();
      f32x16 o;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = 0.0f;
      o = mfma32(as_bf16x8(rtf[0]), as_bf16x8(f[0]), o);
      o = mfma32(as_bf16x8(rtf[1]), as_bf16x8(f[1]), o);
      if constexpr (FP8) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] *= sc[r];
      }
      if (mok) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(dz + (size_t)m * N + nbr + 8 * q + 4 * g2) =
              make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
      }
    }
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

// ---------------------------------------------------------------- dq stage 1, bf16 Y
// The same partial cross products (and rotated copy dz) for bf16 Y, shaped
// for bandwidth: the 64-token x 64-channel tiles of dY and Y travel by
// asynchronous global -> LDS copies (gemm_nt_dma.h) through three LDS
// stages, two steps ahead, in their natural layout; the cross products read
// both operands along the tokens with the LDS transpose load, the rotation
// reads dY rows directly.  The rotated tile is staged in LDS (two buffers)
// and stored one step later as whole 128-byte rows.  Tile row m keeps
// 16-byte chunk c at c ^ f(m),
// f(m) = rot((m >> 1) & 7) (3-bit rotate right): 16 consecutive rows read
// at one chunk fill 16 distinct 16-byte bank slots, and the 4 rows of a
// transpose load use 4 disjoint 32-byte slots.
__device__ __forceinline__ int dqsw(int m) {
  const int x = (m >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

template <bool FP8, int B>
__global__ __launch_bounds__(256, 2) void dq_dma_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ y,
                                                        float* __restrict__ part, int M, int N, int rows_per_split,
                                                        int ng32, const uint16_t* __restrict__ Rops,
                                                        const float* __restrict__ fp8_scale,
                                                        uint16_t* __restrict__ dz, const float* __restrict__ Rf,
                                                        float* __restrict__ dq) {
  using namespace ntd;
  constexpr int ST = 64 * 128;  // bytes per tile
  __shared__ __attribute__((aligned(16))) uint8_t tiles[3][2][ST];  // [stage][dY, Y][m][n]
  __shared__ __attribute__((aligned(16))) uint8_t zt[2][ST];        // rotated tiles, [m][n]
  __shared__ float red[2][64][17];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int n0 = blockIdx.x * 64;
  const int split = blockIdx.y;
  const int m_lo = split * rows_per_split;
  const int m_hi = min(M, m_lo + rows_per_split);
  const int nsteps = (m_hi - m_lo + 63) / 64;
  const bool want_dq = part != nullptr;

  // copies: wave w moves tile rows 16w .. 16w + 15 of dY and of Y (two
  // instructions each, 8 rows x 128 bytes); rows past m_hi copy the tile's
  // first row and columns past N column chunk 0 (neither is used)
  uint32_t off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wave + 8 * i + (lane >> 3);
    const int lc = (lane & 7) ^ dqsw(r);
    const int col = n0 + 8 * lc < N ? n0 + 8 * lc : 0;
    off[i] = (uint32_t)((r * N + col) * 2);
  }
  const uint32_t t_lds = lds_addr(&tiles[0][0][0]) + (uint32_t)(16 * wave * 128);
  auto issue = [&](int s) {
    const int st = s % 3;
    const int m = m_lo + 64 * s;
    const int rows_ok = min(64, m_hi - m);
    uint32_t o[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wave + 8 * i + (lane >> 3);
      o[i] = r < rows_ok ? off[i] : off[i] - (uint32_t)(r * N * 2);  // same column, tile row 0
    }
    const uint16_t* dyb = dy + (size_t)m * N;
    const uint16_t* yb = y + (size_t)m * N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      copy16(t_lds + st * 2 * ST + i * 1024, dyb, o[i]);
      copy16(t_lds + st * 2 * ST + ST + i * 1024, yb, o[i]);
    }
  };

  // rotation of wave (rg, rh): channels n0 + 32 rg, tokens 32 rh of each step
  const int rg = wave & 1, rh = wave >> 1;
  const int nbr = n0 + 32 * rg;
  const bool rot = dz != nullptr && nbr < N;
  bf16x8 rtf[2];
  float sc[16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint4 v = zero4();
    if (rot) {
      if constexpr (B == 32) {
        v = *reinterpret_cast<const uint4*>(Rops + (size_t)(nbr / 32) * 2048 + 1024 + l32 * 32 + 16 * t + 8 * g2);
      } else {
        if ((l32 >> 4) == t)
          v = *reinterpret_cast<const uint4*>(Rops + (size_t)(nbr / 16 + t) * 512 + 256 + (l32 & 15) * 16 + 8 * g2);
      }
    }
    rtf[t] = as_bf16x8(v);
  }
  if constexpr (FP8) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (rot) v = *reinterpret_cast<const float4*>(fp8_scale + nbr + 8 * q + 4 * g2);
      sc[4 * q] = v.x;
      sc[4 * q + 1] = v.y;
      sc[4 * q + 2] = v.z;
      sc[4 * q + 3] = v.w;
    }
  }

  // the rotation operands are in registers before any copy is in flight (a
  // wait the compiler knows about, so it adds none for them in the loop)
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)

  // cross products of wave (grp, kh): channels n0 + 32 grp, token blocks
  // kk = 2 kh, 2 kh + 1 (16 tokens each) of every step
  const int grp = wave & 1, kh = wave >> 1;
  const bool gok = n0 + 32 * grp < N;
  const int G = lane >> 4, li = lane & 15;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  // rows 16 wave .. 16 wave + 15 of the staged rotated tile of step s -> dz
  auto store_z = [&](int s) {
    const int m = m_lo + 64 * s;
    const int rows_ok = min(64, m_hi - m);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wave + 8 * i + (lane >> 3);
      const int c = lane & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(&zt[s & 1][r * 128 + 16 * (c ^ dqsw(r))]);
      if (r < rows_ok && n0 + 8 * c < N) *reinterpret_cast<uint4*>(dz + (size_t)(m + r) * N + n0 + 8 * c) = v;
    }
  };

  issue(0);
  if (nsteps > 1) issue(1);
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) wait_copies_barrier<4>(); else wait_copies_barrier<0>();
    const int st = s % 3;
    const uint8_t* T = &tiles[st][0][0];
    const int rows_ok = min(64, m_hi - (m_lo + 64 * s));  // valid tokens of this step
    if (dz != nullptr && s > 0) store_z(s - 1);
    if (rot) {
      // dZ^T = R^T dY^T: B operand = dY row (token 32 rh + l32), channels
      // nbr + 16 t + 8 g2 .. + 7; the result (channels 32 rg + 8 q + 4 g2
      // .. + 3 of that token) goes to the staging tile
      const int r = 32 * rh + l32;
      f32x16 o;
#pragma unroll
      for (int q = 0; q < 16; ++q) o[q] = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int lc = (32 * rg + 16 * t + 8 * g2) / 8;
        const bf16x8 f = *reinterpret_cast<const bf16x8*>(T + r * 128 + 16 * (lc ^ dqsw(r)));
        o = mfma32(rtf[t], f, o);
      }
      if constexpr (FP8) {
#pragma unroll
        for (int q = 0; q < 16; ++q) o[q] *= sc[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2*>(&zt[s & 1][r * 128 + 16 * ((4 * rg + q) ^ dqsw(r)) + 8 * g2]) =
            make_uint2(pack_bf16x2(o[4 * q], o[4 * q + 1]), pack_bf16x2(o[4 * q + 2], o[4 * q + 3]));
    }
    // the dz stores above precede these copies: at the next barrier the 4
    // copies of step s + 2, if any, are the youngest of this wave's loads
    // and stores, and everything older (the copies of step s + 1) must land
    if (s + 2 < nsteps) issue(s + 2);
    if (want_dq && gok) {
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const int kk = 2 * kh + kq;
        // lane (li, G): tile rows 16 kk + 8 (G >> 1) + li / 4 (+ 4), channel
        // 32 grp + 16 (G & 1) + 4 (li & 3): it receives channel + li's four
        // tokens, i.e. operand row l32, items 8 g2 .. 8 g2 + 7
        const int col = 32 * grp + 16 * (G & 1) + 4 * (li & 3);
        const int r0 = 16 * kk + 8 * (G >> 1) + (li >> 2);
        uint2 d[2], yv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = r0 + 4 * h;
          const int boff = r * 128 + 16 * ((col / 8) ^ dqsw(r)) + 2 * (col % 8);
          d[h] = nn::ds_read_tr16(reinterpret_cast<const uint16_t*>(T + boff));
          yv[h] = nn::ds_read_tr16(reinterpret_cast<const uint16_t*>(T + ST + boff));
        }
        uint4 a = make_uint4(d[0].x, d[0].y, d[1].x, d[1].y);
        const uint4 b = make_uint4(yv[0].x, yv[0].y, yv[1].x, yv[1].y);
        if (16 * kk + 16 > rows_ok) {
          // ragged last step: this lane's tokens 16 kk + 8 g2 + p past the slice end contribute 0
          const int base = 16 * kk + 8 * g2;
          uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int pp = 0; pp < 8; ++pp)
            if (base + pp >= rows_ok) w[pp >> 1] &= (pp & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          a = make_uint4(w[0], w[1], w[2], w[3]);
        }
        acc = mfma32(as_bf16x8(a), as_bf16x8(b), acc);
      }
    }
  }
  if (dz != nullptr) {
    lds_barrier_plain();
    store_z(nsteps - 1);
  }
  if (!want_dq) return;

  // fixed-order reduction of the two token halves, then one partial per slice
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[grp][lane][r] = acc[r];
  }
  __syncthreads();
  if (dq == nullptr) {
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
    return;
  }
  // one slice (few tokens): the workgroup holds the whole S of its 64
  // channels and finishes their blocks itself (the tiles are free now)
  float(*Sg)[32][33] = reinterpret_cast<float(*)[32][33]>(&tiles[0][0][0]);
  if (kh == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) Sg[grp][(r / 4) * 8 + 4 * g2 + (r % 4)][l32] = acc[r] + red[grp][lane][r];
  }
  __syncthreads();
  constexpr int GB = 1024 / (B * B), NP = B * (B - 1) / 2;
  float* scratch = reinterpret_cast<float*>(&tiles[1][0][0]);  // 32 KB free past Sg
  const int nblk = N / B;
  if constexpr (B == 32) {
    // the two blocks at once on the fp32 matrix cores, wave w < 2 taking
    // block w: T1 = S + S R (D = A B + C with A = S, B = R, C = S), then
    // 2 Gq = T1 + R^T T1 (A = R^T, B = T1, C = T1); in step s of
    // v_mfma_f32_32x32x2f32 lane (l32, g2) supplies A[l32][2 s + g2] and
    // B[2 s + g2][l32], and holds D[8 (r / 4) + 4 g2 + r % 4][l32] in r
    auto T1 = reinterpret_cast<float(*)[32][33]>(scratch);
    const int jb = n0 / 32 + wave;
    if (wave < 2 && jb < nblk) {
      const float* Rg = Rf + (size_t)jb * 1024;
      float rk[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) rk[s2] = Rg[(2 * s2 + g2) * 32 + l32];
      f32x16 t;
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = Sg[wave][(r / 4) * 8 + 4 * g2 + (r % 4)][l32];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2)
        t = __builtin_amdgcn_mfma_f32_32x32x2f32(Sg[wave][l32][2 * s2 + g2], rk[s2], t, 0, 0, 0);
      // (LDS accesses of one wave complete in order: T1 is read back below,
      // S is overwritten after its last read)
#pragma unroll
      for (int r = 0; r < 16; ++r) T1[wave][(r / 4) * 8 + 4 * g2 + (r % 4)][l32] = t[r];
      f32x16 gq = t;
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2)
        gq = __builtin_amdgcn_mfma_f32_32x32x2f32(rk[s2], T1[wave][2 * s2 + g2][l32], gq, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) Sg[wave][(r / 4) * 8 + 4 * g2 + (r % 4)][l32] = 0.5f * gq[r];
    }
    __syncthreads();
    // dp_il = Gq_il - Gq_li: thread (block tid / 128, row i, columns
    // 8 (tid % 4) .. + 7 above the diagonal), packed index i B - i (i + 1) / 2 + l - i - 1
    const int b2 = tid >> 7, i = (tid & 127) >> 2, c8 = 8 * (tid & 3);
    if (n0 / 32 + b2 < nblk) {
      float* dst = dq + (size_t)(n0 / 32 + b2) * NP + (i * 32 - i * (i + 1) / 2 - i - 1);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int l = c8 + k;
        if (l > i) dst[l] = Sg[b2][i][l] - Sg[b2][l][i];
      }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < 64 / (GB * B); ++q) {
    const int j0 = n0 / B + q * GB;  // first block of the group
    if (j0 >= nblk) break;          // uniform
    cayley_grad_group<B>(scratch, Rf + (size_t)j0 * B * B, dq + (size_t)j0 * NP, min(GB, nblk - j0), tid,
                         [&](int g, int r, int c) {
                           const int ch = (q * GB + g) * B;  // first channel of the block in the tile
                           const float* row = &Sg[ch / 32][ch % 32 + r][ch % 32 + c];
                           return make_float4(row[0], row[1], row[2], row[3]);
                         });
    __syncthreads();
  }
}

// ---------------------------------------------------------------- dq stage 2
// Per block: S = sum of the slice partials (fixed order); with
// R (R^T + I) = I + R the Cayley gradient is
//   Gq = (R^T + I) S (I + R) / 2,  dp_il = Gq_il - Gq_li.
template <int B>
__global__ __launch_bounds__(256) void dq_final_kernel(const float* __restrict__ part, int nsplit, int ng32,
                                                       int nblk, const float* __restrict__ Rf,
                                                       float* __restrict__ dq) {
  constexpr int G = 1024 / (B * B);
  __shared__ __attribute__((aligned(16))) float lds[3 * G * B * (B + 4)];
  const int j0 = blockIdx.x * G;
  cayley_grad_group<B>(lds, Rf + (size_t)j0 * B * B, dq + (size_t)j0 * (B * (B - 1) / 2), min(G, nblk - j0),
                       threadIdx.x, [&](int g, int r, int c) {
                         const int j = j0 + g, g32 = (j * B) / 32, off = (j * B) % 32;
                         const float* src = part + (size_t)g32 * 1024 + (off + r) * 32 + off + c;
                         // every slice load in flight first (nsplit <= 16), then a fixed-order sum
                         float4 v[16];
#pragma unroll
                         for (int sp = 0; sp < 16; ++sp)
                           v[sp] = sp < nsplit ? *reinterpret_cast<const float4*>(src + (size_t)sp * ng32 * 1024)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
                         float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                         for (int sp = 0; sp < 16; ++sp) {
                           s.x += v[sp].x;
                           s.y += v[sp].y;
                           s.z += v[sp].z;
                           s.w += v[sp].w;
                         }
                         return s;
                       });
}

// dx[m][k] = sum_z part[z][m][k] in a fixed order (contraction split)
template <bool XF32>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int nsplit, size_t n4,
                                                           void* __restrict__ dx) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4* src = reinterpret_cast<const float4*>(part) + i;
  // eight slices' loads in flight at a time, then their sum in slice order
  constexpr int CH = 8;
  float4 s = src[0];
  for (int z0 = 1; z0 < nsplit; z0 += CH) {
    float4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (z0 + c < nsplit) v[c] = src[(size_t)(z0 + c) * n4];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (z0 + c < nsplit) {
        s.x += v[c].x;
        s.y += v[c].y;
        s.z += v[c].z;
        s.w += v[c].w;
      }
    }
  }
  if constexpr (XF32) {
    reinterpret_cast<float4*>(dx)[i] = s;
  } else {
    reinterpret_cast<uint2*>(dx)[i] = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
  }
}

template <bool XF32, int WF, int B, int PRO>
hipError_t launch_dx_t(const DenseArgs& a, const DqPlan& pl, const uint16_t* src, const uint8_t* wc,
                       const void* ws, const uint16_t* Rops, void* dx, char* work, hipStream_t st) {
  constexpr int BM = 128;
  constexpr int NB = 1;
  NnArgs p{};
  p.src = src;
  p.lds = a.N;
  p.wc = wc;
  p.ws = ws;
  p.rops = Rops;
  p.out = dx;
  p.ldo = a.K;
  p.M = a.M;
  p.K = a.K;
  p.N = a.N;
  p.g = a.g;
  dim3 grid((a.K + nn::BKO - 1) / nn::BKO, (a.M + BM - 1) / BM, pl.nsplit_n > 1 ? pl.nsplit_n : 1);
  if (pl.nsplit_n > 1) {
    p.nsplit_len = pl.nsplit_len;
    p.part = reinterpret_cast<float*>(work + pl.npart_off);
  }
  {
    ProfScope prof(st, "dense.dx");
    // INT4 on the rotated copy dZ': the codes stream through the copy ring
    // of gemm_nn_q4_kernel (4-bit transpose loads, 256 output columns per
    // workgroup, no transposed or dequantised copy of the weight); few
    // tokens split the contraction, its fp32 partials into the same split
    // sum (the unsplit kernel stores bf16 dX only)
    bool q4 = false;
    if constexpr (WF == WF_INT4 && PRO == PRO_NONE) {
      const bool split_ok = pl.nsplit_n > 1 && pl.nsplit_len % nnq::BNS == 0;
      if (a.K % nnq::BKO == 0 && a.N % nnq::BNS == 0 && (split_ok || (pl.nsplit_n == 1 && !XF32))) {
        const dim3 qgrid(a.K / nnq::BKO, (a.M + nnq::BM - 1) / nnq::BM, pl.nsplit_n);
        hipLaunchKernelGGL((gemm_nn_q4_kernel<EPI_STORE, false, false>), qgrid, dim3(nnq::NTHR), 0, st, p);
        q4 = true;
      }
    }
    if (!q4)
      hipLaunchKernelGGL((gemm_nn_kernel<BM, XF32, WF, B, PRO, EPI_STORE, false, NB>), grid, dim3(256), 0, st, p);
  }
  if (pl.nsplit_n > 1) {
    ProfScope prof(st, "dense.dx_reduce");
    const size_t n4 = (size_t)a.M * a.K / 4;
    hipLaunchKernelGGL(split_reduce_kernel<XF32>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, p.part,
                       pl.nsplit_n, n4, dx);
  }
  return hipGetLastError();
}


// ---------------------------------------------------------------- transposed weight
// FP8 codes [N][K] -> [K][N], 64 x 64 tiles: rows go through LDS as 4-byte
// words, each thread transposes a 4 x 4 byte block in registers.
__global__ __launch_bounds__(256) void transpose_fp8_kernel(const uint8_t* __restrict__ in,
                                                            uint8_t* __restrict__ out, int N, int K) {
  __shared__ uint32_t t[64][17];
  const int tid = threadIdx.x;
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  {
    const int n = tid >> 2, q = tid & 3;
    const uint4 v = *reinterpret_cast<const uint4*>(in + (size_t)(n0 + n) * K + k0 + 16 * q);
    t[n][4 * q] = v.x;
    t[n][4 * q + 1] = v.y;
    t[n][4 * q + 2] = v.z;
    t[n][4 * q + 3] = v.w;
  }
  __syncthreads();
  const int bn = tid & 15, bk = tid >> 4;  // 4 x 4 block: n 4bn.., k 4bk..
  const uint32_t w0 = t[4 * bn][bk], w1 = t[4 * bn + 1][bk], w2 = t[4 * bn + 2][bk], w3 = t[4 * bn + 3][bk];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t o = ((w0 >> (8 * j)) & 0xFFu) | (((w1 >> (8 * j)) & 0xFFu) << 8) |
                       (((w2 >> (8 * j)) & 0xFFu) << 16) | (((w3 >> (8 * j)) & 0xFFu) << 24);
    *reinterpret_cast<uint32_t*>(out + (size_t)(k0 + 4 * bk + j) * N + n0 + 4 * bn) = o;
  }
}

// 4-bit codes [N][K/2] + group scales [N][K/g] -> bf16 [K][N] holding the
// dequant hook's values; 64 x 64 tiles, natural layout in LDS, each thread
// then pairs two rows n into 4-byte output words.
template <int WF>
__global__ __launch_bounds__(256) void transpose_dequant_w4_kernel(const uint8_t* __restrict__ codes,
                                                                     const uint16_t* __restrict__ scales,
                                                                     uint16_t* __restrict__ out, int N, int K,
                                                                     int g) {
  constexpr int LD = 64 + 8;  // bf16 per LDS row
  __shared__ __attribute__((aligned(16))) uint16_t t[64 * LD];
  const int tid = threadIdx.x;
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  {
    const int n = tid >> 2, q = tid & 3;  // in-features k0 + 16q .. + 15 (one scale group: g >= 32)
    const uint2 c = *reinterpret_cast<const uint2*>(codes + (size_t)(n0 + n) * (K / 2) + (k0 + 16 * q) / 2);
    const auto sc = W4<WF>::scale(scales[(size_t)(n0 + n) * (K / g) + (k0 + 16 * q) / g]);
    uint4* dst = reinterpret_cast<uint4*>(&t[n * LD + 16 * q]);
    dst[0] = W4<WF>::dq(c.x, sc);
    dst[1] = W4<WF>::dq(c.y, sc);
  }
  __syncthreads();
  const int np = tid & 31, kq = tid >> 5;  // rows n 2np, 2np + 1; in-features 8kq .. 8kq + 7
  const uint4 r0 = *reinterpret_cast<const uint4*>(&t[(2 * np) * LD + 8 * kq]);
  const uint4 r1 = *reinterpret_cast<const uint4*>(&t[(2 * np + 1) * LD + 8 * kq]);
  const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w}, b[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t base = (size_t)(k0 + 8 * kq + 2 * j) * N + n0 + 2 * np;
    *reinterpret_cast<uint32_t*>(out + base) = (a[j] & 0xFFFFu) | (b[j] << 16);
    *reinterpret_cast<uint32_t*>(out + base + N) = (a[j] >> 16) | (b[j] & 0xFFFF0000u);
  }
}

// dX = dZ' . W through the transposed weight (plan.wt)
template <bool XF32, int WF>
hipError_t launch_dx_wt(const DenseArgs& a, const DqPlan& pl, const uint16_t* dz, const uint8_t* wc,
                        const void* ws, void* dx, char* work, hipStream_t st) {
  constexpr bool FP8 = WF == WF_FP8;
  uint8_t* wt = reinterpret_cast<uint8_t*>(work + pl.wt_off);
  const dim3 tgrid(a.K / 64, a.N / 64);
  {
  ProfScope prof(st, "dense.transpose");
  if constexpr (FP8)
    hipLaunchKernelGGL(transpose_fp8_kernel, tgrid, dim3(256), 0, st, wc, wt, a.N, a.K);
  else
    hipLaunchKernelGGL(transpose_dequant_w4_kernel<WF>, tgrid, dim3(256), 0, st, wc,
                       static_cast<const uint16_t*>(ws), reinterpret_cast<uint16_t*>(wt), a.N, a.K, a.g);
  }
  ProfScope prof(st, "dense.dx");
  NtArgs p{};
  p.a = dz;
  p.lda = a.N;
  p.wc = wt;
  p.ws = nullptr;
  p.rops = nullptr;
  p.out = dx;
  p.ldo = a.K;
  p.M = a.M;
  p.K = a.N;  // contraction: the layer's output channels
  p.N = a.K;  // output columns: the layer's input features
  p.g = 64;
  const int ntl = (a.K + ntd::BN - 1) / ntd::BN;
  if constexpr (FP8) {
    const int bm = pick_token_tile(ntl, a.M, num_cus(), 192);
    if (bm == 192 && a.N % 128 == 0)  // 128-wide K steps
      hipLaunchKernelGGL((gemm_nt_dma_kernel<WF_FP8, 32, 192, EPI_PLAIN, XF32, false, 128>),
                         dim3(ntl, (a.M + 191) / 192), dim3(ntd::NTHR), 0, st, p);
    else if (bm == 192)
      hipLaunchKernelGGL((gemm_nt_dma_kernel<WF_FP8, 32, 192, EPI_PLAIN, XF32>), dim3(ntl, (a.M + 191) / 192),
                         dim3(ntd::NTHR), 0, st, p);
    else
      hipLaunchKernelGGL((gemm_nt_dma_kernel<WF_FP8, 32, 128, EPI_PLAIN, XF32>), dim3(ntl, (a.M + 127) / 128),
                         dim3(ntd::NTHR), 0, st, p);
  } else {
    hipLaunchKernelGGL((gemm_nt_dma_kernel<WF_BF16, 32, 128, EPI_PLAIN, XF32>), dim3(ntl, (a.M + 127) / 128),
                       dim3(ntd::NTHR), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace

// workgroups of the split-contraction INT4 dX (few tokens): fewer splits
// mean fewer fp32 partials to write and sum; 192 was the best of 128 .. 1024
// at 64 tokens x 2560 in-features x 19456 channels
constexpr int Q4_SPLIT_WGS = 192;

DqPlan plan_bwd(int M, int K, int N, bool fp8, bool int4, bool xf32) {
  DqPlan p;
  p.ng32 = N / 32;
  const int ng64 = (N + 63) / 64;
  const int msteps = (M + 63) / 64;
  // M slices of the dq pass: fewest (rounds of workgroups x 64-token steps
  // per workgroup), two workgroups per CU, at most 16 slices
  const long slots = 2L * num_cus();
  int best = 1;
  long best_cost = -1;
  for (int ns = 1; ns <= 16 && ns <= msteps; ++ns) {
    const long steps_per = (msteps + ns - 1) / ns;
    const long used = (msteps + steps_per - 1) / steps_per;  // slices actually needed
    const long rounds = ((long)ng64 * used + slots - 1) / slots;
    const long cost = rounds * steps_per;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = ns;
    }
  }
  if (msteps == 0) {
    p.nsplit = 0;
    p.rows_per_split = 64;
  } else {
    const int steps_per = (msteps + best - 1) / best;
    p.rows_per_split = steps_per * 64;
    p.nsplit = (msteps + steps_per - 1) / steps_per;
  }
  p.part_bytes = (size_t)(p.nsplit > 0 ? p.nsplit : 1) * p.ng32 * 1024 * sizeof(float);
  // Wide layers rotate dY once in the dQ pass; narrow ones (at most two
  // 128-column tiles of dX) keep the rotation in the dX GEMM prologue.
  p.prerotate = K > 2 * nn::BKO;
  p.dz_off = (p.part_bytes + 255) / 256 * 256;
  size_t end = p.dz_off + (p.prerotate ? (size_t)M * N * 2 : 0);
  // Few tokens: the dX GEMM has (K / 128) x 1 tiles only; split its
  // contraction so that about 512 workgroups stream the weight, each
  // writing an fp32 partial reduced afterwards in a fixed order.
  p.nsplit_n = 1;
  p.nsplit_len = 0;
  p.npart_off = 0;
  // (INT4 with K % 256 == 0 and N % 64 == 0 runs gemm_nn_q4_kernel: 256
  // columns per workgroup)
  const bool q4 = int4 && K % nnq::BKO == 0 && N % nnq::BNS == 0;
  const int ktiles = q4 ? K / nnq::BKO : (K + nn::BKO - 1) / nn::BKO;
  const int target = q4 ? Q4_SPLIT_WGS : 512;
  if (M > 0 && M <= 128 && p.prerotate) {
    int want = (target + ktiles - 1) / ktiles;
    const int nsteps = (N + nn::BNS - 1) / nn::BNS;
    if (want > nsteps) want = nsteps;
    if (want > 1) {
      const int steps_per = (nsteps + want - 1) / want;
      p.nsplit_len = steps_per * nn::BNS;
      p.nsplit_n = (N + p.nsplit_len - 1) / p.nsplit_len;
      p.npart_off = (end + 255) / 256 * 256;
      end = p.npart_off + (size_t)p.nsplit_n * M * K * 4;
    }
  }
  // Wide layer, many tokens: transposed weight for gemm_nt_dma_kernel
  // (FP8 codes, or FP4 / fp32-x INT4 dequantised to bf16); INT4 with bf16 x
  // reads its codes in place on gemm_nn_q4_kernel instead
  p.wt = M > 0 && p.prerotate && p.nsplit_n == 1 && N % 64 == 0 && !(q4 && !xf32);
  p.wt_off = 0;
  if (p.wt) {
    p.wt_off = (end + 255) / 256 * 256;
    end = p.wt_off + (size_t)K * N * (fp8 ? 1 : 2);
  }
  p.bytes = end;
  return p;
}

hipError_t launch_linear_bwd(const DenseArgs& a, const DqPlan& p, const uint16_t* dy, const void* y,
                             const uint8_t* wc, const void* ws, const float* Rf, const uint16_t* Rops,
                             void* dx, float* dq, char* work, hipStream_t st) {
  float* part = reinterpret_cast<float*>(work);
  uint16_t* dz = (dx != nullptr && p.prerotate && a.M > 0) ? reinterpret_cast<uint16_t*>(work + p.dz_off) : nullptr;
  if ((dq != nullptr || dz != nullptr) && p.nsplit > 0) {
    ProfScope prof(st, "dense.dq");
    dim3 grid((a.N + 63) / 64, p.nsplit);
    const float* s8 = a.fp8 ? static_cast<const float*>(ws) : nullptr;
    float* dq_part = dq != nullptr ? part : nullptr;
    // one slice: the dq pass finishes the blocks itself (no dq_final launch)
    float* dq_fused = (dq != nullptr && p.nsplit == 1) ? dq : nullptr;
#define OFT_DQD(F8, BB)                                                                                   \
  if (!a.xf32 && a.fp8 == F8 && a.b == BB)                                                                \
    hipLaunchKernelGGL((dq_dma_kernel<F8, BB>), grid, dim3(256), 0, st, dy, static_cast<const uint16_t*>(y), \
                       dq_part, a.M, a.N, p.rows_per_split, p.ng32, Rops, s8, dz, Rf, dq_fused);
    OFT_DQD(false, 32)
    OFT_DQD(false, 16)
    OFT_DQD(true, 32)
    OFT_DQD(true, 16)
#undef OFT_DQD
#define OFT_DQP(F8, BB)                                                                                   \
  if (a.xf32 && a.fp8 == F8 && a.b == BB)                                                                 \
    hipLaunchKernelGGL((dq_partial_kernel<true, F8, BB>), grid, dim3(256), 0, st, dy, y, part, a.M, a.N,  \
                       p.rows_per_split, p.ng32, Rops, s8, dz);
    OFT_DQP(false, 32)
    OFT_DQP(false, 16)
    OFT_DQP(true, 32)
    OFT_DQP(true, 16)
#undef OFT_DQP
  }
  const bool fused = dq != nullptr && p.nsplit == 1 && !a.xf32;
  if (dq != nullptr && !fused) {
    ProfScope prof(st, "dense.dq_final");
    const int nblk = a.N / a.b;
    if (a.b == 32)
      hipLaunchKernelGGL(dq_final_kernel<32>, dim3(nblk), dim3(256), 0, st, part, p.nsplit, p.ng32, nblk, Rf, dq);
    else
      hipLaunchKernelGGL(dq_final_kernel<16>, dim3((nblk + 3) / 4), dim3(256), 0, st, part, p.nsplit, p.ng32,
                         nblk, Rf, dq);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || dx == nullptr || a.M == 0) return err;
  if (dz != nullptr && p.wt) {
#define OFT_DXW(XF, WFV) \
  if (a.xf32 == XF && a.wf == WFV) return launch_dx_wt<XF, WFV>(a, p, dz, wc, ws, dx, work, st);
    OFT_DXW(false, WF_INT4)
    OFT_DXW(false, WF_FP8)
    OFT_DXW(false, WF_FP4)
    OFT_DXW(true, WF_INT4)
    OFT_DXW(true, WF_FP8)
    OFT_DXW(true, WF_FP4)
#undef OFT_DXW
    return hipErrorInvalidValue;
  }
#define OFT_DX(XF, WFV, BB)                                                                             \
  if (a.xf32 == XF && a.wf == WFV && a.b == BB)                                                         \
    return dz != nullptr ? launch_dx_t<XF, WFV, BB, PRO_NONE>(a, p, dz, wc, ws, Rops, dx, work, st)    \
                         : launch_dx_t<XF, WFV, BB, PRO_ROT>(a, p, dy, wc, ws, Rops, dx, work, st);
#define OFT_DX_B(XF, WFV) OFT_DX(XF, WFV, 32) OFT_DX(XF, WFV, 16)
  OFT_DX_B(false, WF_INT4)
  OFT_DX_B(false, WF_FP8)
  OFT_DX_B(false, WF_FP4)
  OFT_DX_B(true, WF_INT4)
  OFT_DX_B(true, WF_FP8)
  OFT_DX_B(true, WF_FP4)
#undef OFT_DX_B
#undef OFT_DX
  return hipErrorInvalidValue;
}

}  // namespace oft
