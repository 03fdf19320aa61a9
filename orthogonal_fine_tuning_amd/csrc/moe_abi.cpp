// extern "C" MoE entry points of liboft (declared in include/oft.h).
// Arguments are validated on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include "oft.h"
#include "oft_launch.h"
#include "oft_moe.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }

int32_t validate_moe(const oft_moe_desc* d) {
  if (d == nullptr) return OFT_EINVAL;
  if (d->T < 0 || d->E <= 0 || d->k <= 0 || d->H <= 0 || d->I <= 0 || d->chunk < 1) return OFT_EINVAL;
  if (d->k > 16 || d->E > 1024 || d->k > d->E) return OFT_EUNSUPPORTED;
  // the grouped work lists run along grid y (at most 65535 workgroups): the
  // finest, 16-row tiles of the few-rows-per-expert forward, number at most
  // ceil(T k / 16) + E
  if (d->H > (1 << 16) || d->I > (1 << 16)) return OFT_EUNSUPPORTED;
  if (((long long)d->T * d->k + 15) / 16 + d->E > 65535) return OFT_EUNSUPPORTED;
  if (d->b != 16 && d->b != 32) return OFT_EUNSUPPORTED;
  if (d->w_fmt != OFT_W_INT4 && d->w_fmt != OFT_W_INT4_TILED && d->w_fmt != OFT_W_FP4_E2M1 &&
      d->w_fmt != OFT_W_BF16)
    return OFT_EDTYPE;
  if ((long long)d->I * d->H >= (1LL << 31)) return OFT_EUNSUPPORTED;
  const bool w4 = d->w_fmt != OFT_W_BF16;  // INT4 (either storage) or FP4: codes + group scales
  if (w4 && d->g != 32 && d->g != 64 && d->g != 128) return OFT_EUNSUPPORTED;
  if (d->renorm != 0 && d->renorm != 1) return OFT_EINVAL;
  if (d->H % 64 != 0 || d->I % 64 != 0 || d->I % d->b != 0) return OFT_ESHAPE;
  if (w4 && (d->H % d->g != 0 || d->I % d->g != 0)) return OFT_ESHAPE;
  // tiled storage: the kernels that read it take 256-wide K steps (dec4,
  // the NN backward) on both matrices
  if (d->w_fmt == OFT_W_INT4_TILED && (d->H % 256 != 0 || d->I % 256 != 0)) return OFT_ESHAPE;
  return OFT_OK;
}

oft::MoeDims dims(const oft_moe_desc* d) {
  const int wf = d->w_fmt == OFT_W_INT4         ? oft::WF_INT4
                 : d->w_fmt == OFT_W_INT4_TILED ? oft::WF_INT4T
                 : d->w_fmt == OFT_W_FP4_E2M1   ? oft::WF_FP4
                                                : oft::WF_BF16;
  return oft::MoeDims{d->T, d->E, d->k, d->H, d->I, wf != oft::WF_BF16 ? d->g : 64, d->b, d->chunk, d->renorm, wf};
}

// scales are required for the 4-bit formats only
bool scales_ok(const oft_moe_desc* d, const void* p) { return d->w_fmt == OFT_W_BF16 || ptr_ok(p); }

int32_t routing_ok(const oft_moe_routing* rt) {
  if (rt == nullptr) return OFT_EINVAL;
  const void* ptrs[] = {rt->topk_idx, rt->topk_w, rt->counts, rt->offsets, rt->perm,
                        rt->inv_perm, rt->active, rt->n_active, rt->chunk_of_expert};
  for (const void* p : ptrs)
    if (!ptr_ok(p)) return OFT_EINVAL;
  return OFT_OK;
}

oft::MoeRoutingDev routing_dev(const oft_moe_routing* rt) {
  return oft::MoeRoutingDev{rt->topk_idx, rt->topk_w, rt->counts, rt->offsets, rt->perm,
                            rt->inv_perm, rt->active, rt->n_active, rt->chunk_of_expert};
}

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return OFT_OK;
  oft::set_last_hip_error(static_cast<int>(e));
  return OFT_EHIP;
}

}  // namespace

extern "C" {

int32_t oft_moe_workspace_bytes(const oft_moe_desc* d, int32_t pass, size_t* bytes) {
  if (bytes == nullptr) return OFT_EINVAL;
  const int32_t v = validate_moe(d);
  if (v != OFT_OK) return v;
  if (pass != OFT_PASS_FWD && pass != OFT_PASS_BWD) return OFT_EINVAL;
  *bytes = oft::moe_ws_layout(dims(d), pass).bytes;
  return OFT_OK;
}

int32_t oft_moe_route(const oft_moe_desc* d, const float* logits, const oft_moe_routing* rt, void* ws,
                      size_t ws_bytes, void* stream) {
  int32_t v = validate_moe(d);
  if (v != OFT_OK) return v;
  if ((v = routing_ok(rt)) != OFT_OK) return v;
  if (d->T > 0 && !ptr_ok(logits)) return OFT_EINVAL;
  const oft::MoeWs L = oft::moe_ws_layout(dims(d), OFT_PASS_FWD);
  if (!ptr_ok(ws)) return OFT_EINVAL;
  if (ws_bytes < L.bytes) return OFT_EWORKSPACE;
  return hip_status(oft::launch_moe_route(dims(d), logits, routing_dev(rt), static_cast<char*>(ws), L,
                                          static_cast<hipStream_t>(stream)));
}

int32_t oft_moe_router_bwd(const oft_moe_desc* d, const float* logits, const int32_t* topk_idx,
                           const float* dw, float* d_logits, void* stream) {
  const int32_t v = validate_moe(d);
  if (v != OFT_OK) return v;
  if (d->T == 0) return OFT_OK;
  if (!ptr_ok(logits) || !ptr_ok(topk_idx) || !ptr_ok(dw) || !ptr_ok(d_logits)) return OFT_EINVAL;
  return hip_status(oft::launch_moe_router_bwd(dims(d), logits, topk_idx, dw, d_logits,
                                               static_cast<hipStream_t>(stream)));
}

int32_t oft_moe_grouped_fwd(const oft_moe_desc* d, const uint16_t* x, const float* logits,
                            const uint8_t* wgu_codes, const uint16_t* wgu_scales,
                            const uint8_t* wd_codes, const uint16_t* wd_scales,
                            const uint16_t* R_ops, const oft_moe_routing* rt,
                            uint16_t* h_saved, uint16_t* y, void* ws, size_t ws_bytes,
                            void* stream) {
  int32_t v = validate_moe(d);
  if (v != OFT_OK) return v;
  if ((v = routing_ok(rt)) != OFT_OK) return v;
  if (d->T > 0) {
    const void* req[] = {x, logits, wgu_codes, wd_codes, R_ops, h_saved, y};
    for (const void* p : req)
      if (!ptr_ok(p)) return OFT_EINVAL;
    if (!scales_ok(d, wgu_scales) || !scales_ok(d, wd_scales)) return OFT_EINVAL;
  }
  const oft::MoeWs L = oft::moe_ws_layout(dims(d), OFT_PASS_FWD);
  if (!ptr_ok(ws)) return OFT_EINVAL;
  if (ws_bytes < L.bytes) return OFT_EWORKSPACE;
  const oft::MoeFwdPtrs q{x, wgu_codes, wgu_scales, wd_codes, wd_scales, R_ops, h_saved, y};
  return hip_status(oft::launch_moe_fwd(dims(d), logits, q, routing_dev(rt), static_cast<char*>(ws), L,
                                        static_cast<hipStream_t>(stream)));
}

int32_t oft_moe_grouped_fwd_base(const oft_moe_desc* d, const uint16_t* x, const float* logits,
                                 const uint8_t* wgu_codes, const uint16_t* wgu_scales, const uint8_t* wd_codes,
                                 const uint16_t* wd_scales, const oft_moe_routing* rt, uint16_t* h_or_null,
                                 uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  int32_t v = validate_moe(d);
  if (v != OFT_OK) return v;
  if ((v = routing_ok(rt)) != OFT_OK) return v;
  if (!opt_ok(h_or_null)) return OFT_EINVAL;
  if (d->T > 0) {
    const void* req[] = {x, logits, wgu_codes, wd_codes, y};
    for (const void* p : req)
      if (!ptr_ok(p)) return OFT_EINVAL;
    if (!scales_ok(d, wgu_scales) || !scales_ok(d, wd_scales)) return OFT_EINVAL;
  }
  const oft::MoeWs L = oft::moe_ws_layout(dims(d), OFT_PASS_FWD);
  if (!ptr_ok(ws)) return OFT_EINVAL;
  if (ws_bytes < L.bytes) return OFT_EWORKSPACE;
  const oft::MoeFwdPtrs q{x, wgu_codes, wgu_scales, wd_codes, wd_scales, nullptr, h_or_null, y};
  return hip_status(oft::launch_moe_fwd(dims(d), logits, q, routing_dev(rt), static_cast<char*>(ws), L,
                                        static_cast<hipStream_t>(stream), true));
}

int32_t oft_moe_grouped_bwd(const oft_moe_desc* d, const uint16_t* dy, const oft_moe_routing* rt,
                            const uint16_t* h_saved, const uint8_t* wgu_codes,
                            const uint16_t* wgu_scales, const uint8_t* wd_codes,
                            const uint16_t* wd_scales, const float* R_f32,
                            const uint16_t* R_ops, uint16_t* dx_or_null, float* dq_or_null,
                            float* dw_or_null, void* ws, size_t ws_bytes, void* stream) {
  int32_t v = validate_moe(d);
  if (v != OFT_OK) return v;
  if ((v = routing_ok(rt)) != OFT_OK) return v;
  if (!opt_ok(dx_or_null) || !opt_ok(dq_or_null) || !opt_ok(dw_or_null)) return OFT_EINVAL;
  if (dq_or_null != nullptr && !ptr_ok(R_f32)) return OFT_EINVAL;
  if (dx_or_null != nullptr && !ptr_ok(R_ops)) return OFT_EINVAL;
  if (d->T > 0) {
    const void* req[] = {dy, h_saved, wd_codes};
    for (const void* p : req)
      if (!ptr_ok(p)) return OFT_EINVAL;
    if (!scales_ok(d, wd_scales)) return OFT_EINVAL;
    if (dx_or_null != nullptr && (!ptr_ok(wgu_codes) || !scales_ok(d, wgu_scales))) return OFT_EINVAL;
  }
  const oft::MoeWs L = oft::moe_ws_layout(dims(d), OFT_PASS_BWD);
  if (!ptr_ok(ws)) return OFT_EINVAL;
  if (ws_bytes < L.bytes) return OFT_EWORKSPACE;
  const oft::MoeBwdPtrs q{dy, h_saved, wgu_codes, wgu_scales, wd_codes, wd_scales, R_f32, R_ops,
                          dx_or_null, dq_or_null, dw_or_null};
  return hip_status(oft::launch_moe_bwd(dims(d), q, routing_dev(rt), static_cast<char*>(ws), L,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
