// Per-token log-probability difference of two policies (oft_logprob_diff in
// include/oft.h): d[t] = log softmax(a[t])[label[t]] - log softmax(r[t])[label[t]].
//
// The chooseai.io page's "Five design features of the adapter-first
// architecture" regularises the trained policy (base + OFT adapter) towards
// a reference policy that is the frozen base itself, run without the
// adapter; the KL estimate needs both policies' log-probabilities of the
// sampled token, which this gives from their logits.
//
// One workgroup of 256 threads per token: each thread keeps a running
// (maximum, sum of exp(v - maximum)) pair for both rows over a strided
// share of the vocabulary; the pairs are merged by wavefront butterflies and
// then across the four waves, in a fixed order (deterministic).
#include <math.h>

#include "oft_launch.h"
#include "oft_prof.h"

namespace oft {
namespace {

// (m, s) <- the pair of the union of the two sets (s = sum exp(v - m))
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  if (m2 > m) {
    s = s * __expf(m - m2) + s2;
    m = m2;
  } else {
    s += s2 * __expf(m2 - m);
  }
}

__global__ __launch_bounds__(256) void logprob_diff_kernel(const float* __restrict__ a, const float* __restrict__ r,
                                                           const int* __restrict__ labels, int V,
                                                           float* __restrict__ out) {
  __shared__ float red[4][4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* ra = a + (size_t)t * V;
  const float* rr = r + (size_t)t * V;
  float ma = -INFINITY, sa = 0.0f, mr = -INFINITY, sr = 0.0f;
  for (int i = tid; i < V; i += 256) {
    lse_merge(ma, sa, ra[i], 1.0f);
    lse_merge(mr, sr, rr[i], 1.0f);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ma2 = __shfl_xor(ma, off), sa2 = __shfl_xor(sa, off);
    const float mr2 = __shfl_xor(mr, off), sr2 = __shfl_xor(sr, off);
    lse_merge(ma, sa, ma2, sa2);
    lse_merge(mr, sr, mr2, sr2);
  }
  if (lane == 0) {
    red[wave][0] = ma;
    red[wave][1] = sa;
    red[wave][2] = mr;
    red[wave][3] = sr;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) {
      lse_merge(ma, sa, red[w][0], red[w][1]);
      lse_merge(mr, sr, red[w][2], red[w][3]);
    }
    const int lab = labels[t];
    out[t] = (lab >= 0 && lab < V) ? (ra[lab] - (ma + __logf(sa))) - (rr[lab] - (mr + __logf(sr))) : NAN;
  }
}

}  // namespace

hipError_t launch_logprob_diff(int T, int V, const float* a, const float* r, const int* labels, float* out,
                               hipStream_t st) {
  if (T == 0) return hipSuccess;
  ProfScope prof(st, "policy.logprob_diff");
  hipLaunchKernelGGL(logprob_diff_kernel, dim3(T), dim3(256), 0, st, a, r, labels, V, out);
  return hipGetLastError();
}

}  // namespace oft
