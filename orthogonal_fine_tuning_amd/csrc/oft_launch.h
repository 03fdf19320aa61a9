// Internal launchers (host side).  Arguments are validated by the C-ABI
// layer (abi.cpp) before any of these is called; each returns the
// hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oft {

// thread-local hipError_t reported by oft_last_hip_error()
void set_last_hip_error(int e);

// compute units of the current device (queried once per device)
int num_cus();
// Token tile of gemm_nt_dma_kernel: the candidate with the least estimated
// time, rounds of workgroups x tile rows x workgroups per CU / per-tile
// efficiency.  192-token tiles run one workgroup per CU, 128-token tiles two
// (FP8 and INT4 weights; measured rates relative to one 256-token tile per
// CU: 0.95 at 192 tokens, 1.02 for two 128-token tiles, so a 256-token tile
// never wins and is not built).  max_bm limits the choice (bf16 weights:
// 128, one workgroup per CU at 0.88).
inline int pick_token_tile(long col_tiles, long M, int cus, int max_bm) {
  const int cand[2] = {192, 128};
  const bool w16 = max_bm < 192;
  const int per_cu[2] = {1, w16 ? 1 : 2};
  const double eff[2] = {0.95, w16 ? 0.88 : 1.02};
  int best = 128;
  double best_cost = 0.0;
  for (int i = 0; i < 2; ++i) {
    if (cand[i] > max_bm) continue;
    const long tiles = col_tiles * ((M + cand[i] - 1) / cand[i]);
    const long slots = (long)cus * per_cu[i];
    const long rounds = (tiles + slots - 1) / slots;
    const double cost = (double)rounds * cand[i] * per_cu[i] / eff[i];
    if (best_cost == 0.0 || cost < best_cost) {
      best = cand[i];
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_cayley(const uint16_t* q, int nblk, int b, float* Rf, uint16_t* Rops,
                         hipStream_t st);

// fmt: a WF_* value (numbered as the OFT_W_* formats of the C ABI)
hipError_t launch_dequant(int fmt, int rows, int cols, int g, const uint8_t* codes,
                          const void* scales, uint16_t* out, hipStream_t st);
hipError_t launch_pack_t4(int count, int rows, int cols, int g, const uint8_t* codes, const uint16_t* scales,
                          uint8_t* codes_t, uint16_t* scales_t, hipStream_t st);

// Dense layer.  xf32: x / y / dx are fp32 (else bf16); wf: the weight
// format (the 4-bit ones with group g).
struct DenseArgs {
  int M, K, N, g, b;
  bool xf32, fp8;  // fp8: wf == WF_FP8
  int wf;          // WF_INT4, WF_FP8 or WF_FP4
  // double-buffered adapter (forward only): *rops_sel picks the rotation
  // pack passed to the launch (0) or the one rops_alt elements after it (1)
  long rops_alt = 0;
  const int* rops_sel = nullptr;
};

hipError_t launch_linear_fwd(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws,
                             const uint16_t* Rops, void* y, hipStream_t st);
// adapter slots: state int32[2] = {active slot, its version}, stored and
// loaded as one 64-bit word
hipError_t launch_slots_switch(int* state, int slot, int version, hipStream_t st);
// forward on the active slot: latch int32[2] <- {active, its version}, then
// the forward with a.rops_sel = latch over (R0, R1)
hipError_t launch_linear_fwd_slots(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws,
                                   const uint16_t* R0, const uint16_t* R1, const int* state, int* latch, void* y,
                                   hipStream_t st);
// the frozen base alone: y = x . dequant(W0)^T
hipError_t launch_linear_fwd_base(const DenseArgs& a, const void* x, const uint8_t* wc, const void* ws, void* y,
                                  hipStream_t st);

// Backward plan: split of the M reduction used by dq (deterministic
// partials) and the workspace layout.
struct DqPlan {
  int nsplit;          // number of M slices
  int rows_per_split;  // multiple of 64
  int ng32;            // N / 32 column groups
  size_t part_bytes;   // fp32 partial sums, nsplit * ng32 * 32 * 32 * 4
  bool prerotate;      // dX reads a rotated copy of dY made by the dq pass
  size_t dz_off;       // workspace offset of that copy (bf16 [M, N])
  int nsplit_n;        // contraction splits of the dX GEMM (1 = none)
  int nsplit_len;      // weight rows per split
  size_t npart_off;    // workspace offset of the fp32 dX partials
  bool wt;             // dX runs on a transposed copy of the weight
  size_t wt_off;       // its workspace offset ([K, N]: FP8 codes or bf16)
  size_t bytes;        // total workspace
};
DqPlan plan_bwd(int M, int K, int N, bool fp8, bool int4, bool xf32);

hipError_t launch_linear_bwd(const DenseArgs& a, const DqPlan& p, const uint16_t* dy, const void* y,
                             const uint8_t* wc, const void* ws, const float* Rf, const uint16_t* Rops,
                             void* dx, float* dq, char* work, hipStream_t st);

// per-token log-probability difference of two policies' logits [T, V]
hipError_t launch_logprob_diff(int T, int V, const float* a, const float* r, const int* labels, float* out,
                               hipStream_t st);

}  // namespace oft
