// Cayley build (adapter parameters -> block rotations) and the dequant hook.
//
// Cayley map: the Orbit pages (chooseai.io release news, "Technical
// principles" and "Architectural advantages of OFT over LoRA") make every
// sub-projection's rotation orthogonal; this library builds each b x b block
// as R = (I + Q)(I - Q)^-1 = 2 (I - Q)^-1 - I from the skew-symmetric Q.
//
// Layout of the solve.  Few blocks (cayley_kernel): one workgroup of 4
// waves per block, to spread each solve over 4 SIMDs; lane c of each wave
// owns column c of the augmented matrix [A | I] (2b <= 64 columns) for the
// b/4 rows of its wave's quarter, in registers.  Each of the b
// Gauss-Jordan pivot steps publishes the pivot row and pivot column through
// LDS (ping-pong slots, one barrier per step) and every lane updates its
// rows.  No pivot search is needed: the symmetric part of A is I, so every
// pivot is >= 1.
#include "oft_device.h"
#include "oft_launch.h"

namespace oft {

template <int B>
__global__ __launch_bounds__(256) void cayley_kernel(const uint16_t* __restrict__ q, int nblk,
                                                     float* __restrict__ Rf,
                                                     uint16_t* __restrict__ Rops) {
  constexpr int NT = 256;
  constexpr int RQ = B / 4;  // rows per wave
  constexpr int NP = B * (B - 1) / 2;
  __shared__ float qs[NP];
  __shared__ float prow[2][2 * B];  // pivot row (2b columns)
  __shared__ float pcol[2][B];      // pivot column (b rows)
  __shared__ float Rt[B][B + 1];    // result, for coalesced stores

  const int blk = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid & 63;   // column of [A | I]
  const int w = tid >> 6;   // row quarter
  const bool colv = c < 2 * B;
  for (int i = tid; i < NP; i += NT) qs[i] = bf16_to_f32(q[(size_t)blk * NP + i]);
  __syncthreads();

  float col[RQ];
#pragma unroll
  for (int u = 0; u < RQ; ++u) {
    const int i = w * RQ + u;
    float v = 0.0f;
    if (c < B) {
      float qic = 0.0f;
      if (i < c) qic = qs[i * B - i * (i + 1) / 2 + (c - i - 1)];
      if (i > c) qic = -qs[c * B - c * (c + 1) / 2 + (i - c - 1)];
      v = (i == c ? 1.0f : 0.0f) - qic;
    } else if (colv) {
      v = (i == c - B) ? 1.0f : 0.0f;
    }
    col[u] = v;
  }

  for (int s = 0; s < B; ++s) {
    const int sl = s & 1;
    const int ws = s / RQ, us = s % RQ;
    // publish the pivot row (owned by wave ws) and the pivot column (lane s)
    if (w == ws && colv) {
      float v = 0.0f;
#pragma unroll
      for (int u = 0; u < RQ; ++u)
        if (u == us) v = col[u];
      prow[sl][c] = v;
    }
    if (c == s) {
#pragma unroll
      for (int u = 0; u < RQ; ++u) pcol[sl][w * RQ + u] = col[u];
    }
    __syncthreads();
    if (colv) {
      const float ps = prow[sl][c] / prow[sl][s];  // new pivot-row entry of this column
#pragma unroll
      for (int u = 0; u < RQ; ++u) {
        const int i = w * RQ + u;
        col[u] = (i == s) ? ps : col[u] - pcol[sl][i] * ps;
      }
    }
  }

  // lanes b..2b-1 hold A^-1; R = 2 A^-1 - I
  if (c >= B && colv) {
    const int j = c - B;
#pragma unroll
    for (int u = 0; u < RQ; ++u) {
      const int i = w * RQ + u;
      Rt[i][j] = 2.0f * col[u] - (i == j ? 1.0f : 0.0f);
    }
  }
  __syncthreads();
  float* Rb = Rf + (size_t)blk * B * B;
  uint16_t* R0 = Rops ? Rops + (size_t)blk * 2 * B * B : nullptr;
  for (int e = tid; e < B * B; e += NT) {
    const int i = e / B, j = e % B;
    const float v = Rt[i][j];
    Rb[e] = v;
    if (R0) {
      R0[e] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);                   // R[i][j]
      R0[B * B + j * B + i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);   // R^T[j][i]
    }
  }
}

// Many blocks: one wave solves 64 / (2b) blocks, lane c owning the whole
// column c of [A | I] in registers, the pivot column broadcast through LDS.
template <int B>
__global__ __launch_bounds__(64) void cayley_wave_kernel(const uint16_t* __restrict__ q, int nblk,
                                                    float* __restrict__ Rf,
                                                    uint16_t* __restrict__ Rops) {
  constexpr int LANES = 2 * B;
  constexpr int PER_WAVE = 64 / LANES;
  __shared__ float pivcol[PER_WAVE][B];
  const int lane = threadIdx.x;
  const int sub = lane / LANES;
  const int c = lane % LANES;
  const int blk = blockIdx.x * PER_WAVE + sub;
  const bool valid = blk < nblk;
  const uint16_t* qb = q + (size_t)(valid ? blk : 0) * (B * (B - 1) / 2);

  float col[B];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    float v;
    if (c < B) {
      // A[i][c] = delta - Q[i][c]; Q[i][c] = p(i,c) above, -p(c,i) below
      float qic = 0.0f;
      if (valid && i < c) qic = bf16_to_f32(qb[i * B - i * (i + 1) / 2 + (c - i - 1)]);
      if (valid && i > c) qic = -bf16_to_f32(qb[c * B - c * (c + 1) / 2 + (i - c - 1)]);
      v = (i == c ? 1.0f : 0.0f) - qic;
    } else {
      v = (i == c - B) ? 1.0f : 0.0f;
    }
    col[i] = v;
  }

#pragma unroll
  for (int s = 0; s < B; ++s) {
    if (c == s) {
#pragma unroll
      for (int i = 0; i < B; ++i) pivcol[sub][i] = col[i];
    }
    __syncthreads();
    const float ps = col[s] / pivcol[sub][s];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (i != s) col[i] -= pivcol[sub][i] * ps;
    }
    col[s] = ps;
    __syncthreads();
  }

  if (!valid || c < B) return;
  const int j = c - B;  // this lane holds column j of A^-1
  float* Rb = Rf + (size_t)blk * B * B;
#pragma unroll
  for (int i = 0; i < B; ++i) Rb[i * B + j] = 2.0f * col[i] - (i == j ? 1.0f : 0.0f);
  if (Rops != nullptr) {
    uint16_t* R0 = Rops + (size_t)blk * 2 * B * B;  // R, row-major
    uint16_t* R1 = R0 + B * B;                      // R^T, row-major
    uint32_t packed[B / 2];
#pragma unroll
    for (int i = 0; i < B; i += 2) {
      packed[i / 2] = pack_bf16x2(2.0f * col[i] - (i == j ? 1.0f : 0.0f),
                                  2.0f * col[i + 1] - (i + 1 == j ? 1.0f : 0.0f));
    }
#pragma unroll
    for (int i = 0; i < B; ++i) R0[i * B + j] = (uint16_t)(packed[i / 2] >> (16 * (i & 1)));
    uint4* dst = reinterpret_cast<uint4*>(R1 + j * B);  // row j of R^T = column j of R
#pragma unroll
    for (int v = 0; v < B / 8; ++v)
      dst[v] = make_uint4(packed[4 * v], packed[4 * v + 1], packed[4 * v + 2], packed[4 * v + 3]);
  }
}

// ---- dequant hook: exactly the bf16 values the matrix cores consume -------
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint32_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales,
                                                           uint4* __restrict__ out, size_t n8,
                                                           int cols, int g) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n8) return;
  const int per_row = cols / 8;
  const size_t r = idx / per_row;
  const int c = (int)(idx % per_row) * 8;
  out[idx] = dq_int4x8(codes[idx], i4scale(scales[r * (size_t)(cols / g) + c / g]));
}

__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint2* __restrict__ codes,
                                                          uint4* __restrict__ out, size_t n8) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n8) return;
  const uint2 w = codes[idx];
  const uint2 lo = dq_fp8x4(w.x), hi = dq_fp8x4(w.y);
  out[idx] = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

hipError_t launch_cayley(const uint16_t* q, int nblk, int b, float* Rf, uint16_t* Rops,
                         hipStream_t st) {
  if (nblk == 0) return hipSuccess;
  if (nblk < 2048) {
    if (b == 32)
      hipLaunchKernelGGL(cayley_kernel<32>, dim3(nblk), dim3(256), 0, st, q, nblk, Rf, Rops);
    else
      hipLaunchKernelGGL(cayley_kernel<16>, dim3(nblk), dim3(256), 0, st, q, nblk, Rf, Rops);
  } else {
    if (b == 32)
      hipLaunchKernelGGL(cayley_wave_kernel<32>, dim3(nblk), dim3(64), 0, st, q, nblk, Rf, Rops);
    else
      hipLaunchKernelGGL(cayley_wave_kernel<16>, dim3((nblk + 1) / 2), dim3(64), 0, st, q, nblk, Rf, Rops);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int rows, int cols, int g, const uint8_t* codes,
                          const void* scales, uint16_t* out, hipStream_t st) {
  const size_t n8 = (size_t)rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n8 + 255) / 256);
  if (fmt == 0) {
    hipLaunchKernelGGL(dequant_int4_kernel, dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const uint32_t*>(codes),
                       static_cast<const uint16_t*>(scales), reinterpret_cast<uint4*>(out), n8,
                       cols, g);
  } else {
    hipLaunchKernelGGL(dequant_fp8_kernel, dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const uint2*>(codes), reinterpret_cast<uint4*>(out), n8);
  }
  return hipGetLastError();
}

}  // namespace oft
