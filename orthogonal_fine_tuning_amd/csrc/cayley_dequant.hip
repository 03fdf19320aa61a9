// Cayley build (adapter parameters -> block rotations) and the dequant hook.
//
// Cayley map: the Orbit pages (chooseai.io release news, "Technical
// principles" and "Architectural advantages of OFT over LoRA") make every
// sub-projection's rotation orthogonal; this library builds each b x b block
// as R = (I + Q)(I - Q)^-1 = 2 (I - Q)^-1 - I from the skew-symmetric Q.
//
// Layout of the solve: in-place Gauss-Jordan on A = I - Q with row
// ownership.  Lane r of a b-lane group holds row r of A in registers, so a
// wave solves 64 / b blocks at once and a block needs b, not 2b, lanes (the
// in-place form keeps the growing inverse in the columns already
// eliminated).  Each pivot step publishes the pivot row through LDS and
// every lane applies one fused multiply-add per element.  No pivot search is
// needed: the symmetric part of A is I, so every pivot is >= 1.
#include <utility>

#include "oft_device.h"
#include "oft_launch.h"

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

template <int B>
__global__ __launch_bounds__(64) void cayley_kernel(const uint16_t* __restrict__ q, int nblk,
                                                    float* __restrict__ Rf, uint16_t* __restrict__ Rops) {
  constexpr int PER = 64 / B;  // blocks per wave
  constexpr int NP = B * (B - 1) / 2;
  constexpr int TP = B + 2;  // row pitch (bf16) of the transpose tile
  // the parameters of the wave's blocks, later the bf16 transpose of R
  constexpr int STAGE = PER * NP * 4 > PER * B * TP * 2 ? PER * NP * 4 : PER * B * TP * 2;
  __shared__ __attribute__((aligned(16))) uint8_t stage[STAGE];
  __shared__ __attribute__((aligned(16))) float prow[PER][B];  // pivot row

  const int lane = threadIdx.x;
  const int sub = lane / B, r = lane % B;
  const int blk0 = blockIdx.x * PER;
  const int nv = min(PER, nblk - blk0);  // blocks of this wave
  const int blk = blk0 + sub;

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
  float a[B];
  const float* qb = qs + sub * NP;
#pragma unroll
  for (int c = 0; c < B; ++c) {
    const int lo = c < r ? c : r, hi = c < r ? r : c;
    const float v = (c == r || sub >= nv) ? 0.0f : qb[lo * B - lo * (lo + 1) / 2 + (hi - lo - 1)];
    a[c] = c == r ? 1.0f : (c > r ? -v : v);
  }
  __syncthreads();  // stage is reused for the transpose at the end

  // one pivot step; the step index is a compile-time constant so that every
  // a[] access stays a register
  auto step = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    if (r == s) {
#pragma unroll
      for (int j = 0; j < B; j += 4)
        *reinterpret_cast<float4*>(&prow[sub][j]) = make_float4(a[j], a[j + 1], a[j + 2], a[j + 3]);
    }
    wave_sync();
    float pr[B];
#pragma unroll
    for (int j = 0; j < B; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&prow[sub][j]);
      pr[j] = v.x;
      pr[j + 1] = v.y;
      pr[j + 2] = v.z;
      pr[j + 3] = v.w;
    }
    // 1 / pivot: hardware reciprocal and one Newton step
    const float piv = pr[s];
    float rp = __builtin_amdgcn_rcpf(piv);
    rp = fmaf(rp, fmaf(-piv, rp, 1.0f), rp);
    // pivot row: a_sj / p; other rows: a_rj - (a_rs / p) a_sj; column s of
    // the inverse: 1 / p on the pivot row, -a_rs / p elsewhere
    const float f = a[s];
    const float g = r == s ? 1.0f - rp : f * rp;
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (j != s) a[j] = fmaf(-g, pr[j], a[j]);
    a[s] = r == s ? rp : -g;
    wave_sync();
  };
  for_each_index(step, std::make_integer_sequence<int, B>{});

  // lane r holds row r of A^-1; R = 2 A^-1 - I
#pragma unroll
  for (int j = 0; j < B; ++j) a[j] = 2.0f * a[j] - (j == r ? 1.0f : 0.0f);
  if (sub < nv) {
    float4* dst = reinterpret_cast<float4*>(Rf + (size_t)blk * B * B + r * B);
#pragma unroll
    for (int j = 0; j < B; j += 4) dst[j / 4] = make_float4(a[j], a[j + 1], a[j + 2], a[j + 3]);
  }
  if (Rops == nullptr) return;
  uint32_t pk[B / 2];
#pragma unroll
  for (int j = 0; j < B; j += 2) pk[j / 2] = pack_bf16x2(a[j], a[j + 1]);
  // R^T through LDS: row r of R in, column r of R (row r of R^T) out
  uint16_t* tt = reinterpret_cast<uint16_t*>(stage) + sub * B * TP;
#pragma unroll
  for (int j = 0; j < B; j += 2) *reinterpret_cast<uint32_t*>(tt + r * TP + j) = pk[j / 2];
  __syncthreads();
  uint32_t pt[B / 2];
#pragma unroll
  for (int j = 0; j < B; j += 2) pt[j / 2] = (uint32_t)tt[j * TP + r] | ((uint32_t)tt[(j + 1) * TP + r] << 16);
  if (sub < nv) {
    uint4* r0 = reinterpret_cast<uint4*>(Rops + (size_t)blk * 2 * B * B + r * B);  // R, row r
    uint4* r1 = reinterpret_cast<uint4*>(Rops + (size_t)blk * 2 * B * B + B * B + r * B);  // R^T, row r
#pragma unroll
    for (int v = 0; v < B / 8; ++v) {
      r0[v] = make_uint4(pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]);
      r1[v] = make_uint4(pt[4 * v], pt[4 * v + 1], pt[4 * v + 2], pt[4 * v + 3]);
    }
  }
}

// The same solve with two lanes per row (lane 2r + h holds columns
// [16h, 16h + 16) of row r): half the pivot-row reads and half the updates
// per lane on the serial chain of b pivot steps, for builds of few blocks,
// where that chain is the whole cost.  PER = 32 / B blocks per wave.
template <int B>
__global__ __launch_bounds__(64) void cayley2_kernel(const uint16_t* __restrict__ q, int nblk,
                                                     float* __restrict__ Rf, uint16_t* __restrict__ Rops) {
  constexpr int PER = 32 / B;  // blocks per wave
  constexpr int HB = B / 2;    // columns per lane
  constexpr int NP = B * (B - 1) / 2;
  constexpr int TP = B + 2;  // row pitch (bf16) of the transpose tile
  constexpr int STAGE = PER * NP * 4 > PER * B * TP * 2 ? PER * NP * 4 : PER * B * TP * 2;
  __shared__ __attribute__((aligned(16))) uint8_t stage[STAGE];
  __shared__ __attribute__((aligned(16))) float prow[PER][B];  // pivot row

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

  auto step = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int hs = s / HB, js = s % HB;  // the lane half and slot holding column s
    if (r == s) {
#pragma unroll
      for (int j = 0; j < HB; j += 4)
        *reinterpret_cast<float4*>(&prow[sub][c0 + j]) = make_float4(a[j], a[j + 1], a[j + 2], a[j + 3]);
    }
    // a_rs: held by the lane of half hs of this row
    const float mine = a[js];
    const float other = __shfl_xor(mine, 1);
    const float f = h == hs ? mine : other;
    wave_sync();
    float pr[HB];
#pragma unroll
    for (int j = 0; j < HB; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&prow[sub][c0 + j]);
      pr[j] = v.x;
      pr[j + 1] = v.y;
      pr[j + 2] = v.z;
      pr[j + 3] = v.w;
    }
    const float piv = prow[sub][s];
    float rp = __builtin_amdgcn_rcpf(piv);
    rp = fmaf(rp, fmaf(-piv, rp, 1.0f), rp);
    const float g = r == s ? 1.0f - rp : f * rp;
#pragma unroll
    for (int j = 0; j < HB; ++j)
      if (h != hs || j != js) a[j] = fmaf(-g, pr[j], a[j]);
    if (h == hs) a[js] = r == s ? rp : -g;
    wave_sync();
  };
  for_each_index(step, std::make_integer_sequence<int, B>{});

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

hipError_t launch_cayley(const uint16_t* q, int nblk, int b, float* Rf, uint16_t* Rops,
                         hipStream_t st) {
  if (nblk == 0) return hipSuccess;
  // few blocks (at most a few per SIMD): the serial pivot chain is the cost,
  // so two lanes per row; many blocks: throughput, one lane per row
  const bool two = nblk <= 4 * num_cus() * (b == 32 ? 1 : 2);
  if (b == 32 && two)
    hipLaunchKernelGGL(cayley2_kernel<32>, dim3(nblk), dim3(64), 0, st, q, nblk, Rf, Rops);
  else if (b == 32)
    hipLaunchKernelGGL(cayley_kernel<32>, dim3((nblk + 1) / 2), dim3(64), 0, st, q, nblk, Rf, Rops);
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
