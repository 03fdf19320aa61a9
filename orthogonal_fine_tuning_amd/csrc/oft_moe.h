// Internal interface of the MoE kernels (host side).  The C ABI layer
// (moe_abi.cpp) validates every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include "oft_formats.h"

namespace oft {

struct MoeDims {
  int T, E, k, H, I, g, b, chunk, renorm;
  int wf;  // WF_INT4, WF_FP4 or WF_BF16 (dequantised reference weights)
};

// device pointers of the routing tables (mirrors oft_moe_routing)
struct MoeRoutingDev {
  int* topk_idx;
  float* topk_w;
  int* counts;
  int* offsets;
  int* perm;
  int* inv_perm;
  int* active;
  int* n_active;
  int* chunk_of_expert;
};

// byte offsets of the scratch buffers inside the caller's workspace
struct MoeWs {
  size_t list, ntiles, gmask, tile_off, act, O, dH, dw_part, dXp, dz;
  size_t list64, ntiles64;  // forward: work list of 64-row tiles (few rows per expert)
  long max_tiles, max_tiles64;
  size_t bytes;
};
MoeWs moe_ws_layout(const MoeDims& d, int pass);

struct MoeFwdPtrs {
  const uint16_t* x;
  const uint8_t* wgu_codes;
  const uint16_t* wgu_scales;
  const uint8_t* wd_codes;
  const uint16_t* wd_scales;
  const uint16_t* R_ops;
  uint16_t* h_saved;
  uint16_t* y;
};

struct MoeBwdPtrs {
  const uint16_t* dy;
  const uint16_t* h_saved;
  const uint8_t* wgu_codes;
  const uint16_t* wgu_scales;
  const uint8_t* wd_codes;
  const uint16_t* wd_scales;
  const float* R_f32;
  const uint16_t* R_ops;
  uint16_t* dx;
  float* dq;
  float* dw;
};

hipError_t launch_moe_route(const MoeDims& d, const float* logits, const MoeRoutingDev& rt, char* ws,
                            const MoeWs& L, hipStream_t st);
// base: the frozen base alone (gate/up without the rotation; R_ops unused,
// h_saved optional)
hipError_t launch_moe_fwd(const MoeDims& d, const float* logits, const MoeFwdPtrs& q,
                          const MoeRoutingDev& rt, char* ws, const MoeWs& L, hipStream_t st, bool base = false);
hipError_t launch_moe_bwd(const MoeDims& d, const MoeBwdPtrs& q, const MoeRoutingDev& rt, char* ws,
                          const MoeWs& L, hipStream_t st);
// d_logits [T, E] from dw [T, k] through the softmax and the top-k selection
hipError_t launch_moe_router_bwd(const MoeDims& d, const float* logits, const int* topk_idx, const float* dw,
                                 float* d_logits, hipStream_t st);

}  // namespace oft
