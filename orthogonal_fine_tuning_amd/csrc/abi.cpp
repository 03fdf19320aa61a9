// extern "C" entry points of liboft (declared in include/oft.h).
//
// Every call validates its arguments on the host first; only then does it
// touch the HIP runtime.  On a validation error nothing is enqueued and no
// output is written.
#include <hip/hip_runtime.h>

#include "oft.h"
#include "oft_formats.h"
#include "oft_launch.h"

namespace {

thread_local int g_last_hip = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return OFT_OK;
  g_last_hip = static_cast<int>(e);
  return OFT_EHIP;
}

bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }

static_assert(oft::WF_INT4 == OFT_W_INT4 && oft::WF_FP8 == OFT_W_FP8_E4M3 && oft::WF_BF16 == OFT_W_BF16 &&
                  oft::WF_FP4 == OFT_W_FP4_E2M1 && oft::WF_INT4T == OFT_W_INT4_TILED,
              "kernel weight formats are numbered as the ABI's");

// the 4-bit formats: codes two per byte plus a 16-bit scale per group of g
bool w4(int f) { return f == OFT_W_INT4 || f == OFT_W_FP4_E2M1; }

int32_t validate_linear(const oft_linear_desc* d) {
  if (d == nullptr) return OFT_EINVAL;
  if (d->M < 0 || d->K <= 0 || d->N <= 0) return OFT_EINVAL;
  // index range of the kernels: token tiles of 128 run along grid y (at
  // most 65535 workgroups), and weight element / scale offsets are 32-bit
  // (N K < 2^31 keeps N K / g fp16 scale bytes far inside as well)
  if (d->M > (1 << 22) || d->K > (1 << 20) || d->N > (1 << 20)) return OFT_EUNSUPPORTED;
  if ((long long)d->N * d->K >= (1LL << 31)) return OFT_EUNSUPPORTED;
  if (d->x_dtype != OFT_DT_BF16 && d->x_dtype != OFT_DT_F32) return OFT_EDTYPE;
  if (!w4(d->w_fmt) && d->w_fmt != OFT_W_FP8_E4M3) return OFT_EDTYPE;
  if (d->b != 16 && d->b != 32) return OFT_EUNSUPPORTED;
  if (d->n_seg < 1 || d->n_seg > OFT_MAX_SEGMENTS) return OFT_EUNSUPPORTED;
  long long sum = 0;
  for (int s = 0; s < d->n_seg; ++s) {
    if (d->seg[s] <= 0 || d->seg[s] % d->b != 0) return OFT_ESHAPE;
    sum += d->seg[s];
  }
  if (sum != d->N) return OFT_ESHAPE;
  if (d->N % 32 != 0 || d->K % 64 != 0) return OFT_ESHAPE;
  if (w4(d->w_fmt)) {
    if (!group_ok(d->g)) return OFT_EUNSUPPORTED;
    if (d->K % d->g != 0) return OFT_ESHAPE;
  }
  return OFT_OK;
}

oft::DenseArgs dense_args(const oft_linear_desc* d) {
  oft::DenseArgs a;
  a.M = d->M;
  a.K = d->K;
  a.N = d->N;
  a.g = w4(d->w_fmt) ? d->g : 0;
  a.b = d->b;
  a.xf32 = d->x_dtype == OFT_DT_F32;
  a.fp8 = d->w_fmt == OFT_W_FP8_E4M3;
  a.wf = d->w_fmt == OFT_W_INT4 ? oft::WF_INT4 : a.fp8 ? oft::WF_FP8 : oft::WF_FP4;
  return a;
}

}  // namespace

namespace oft {
void set_last_hip_error(int e) { g_last_hip = e; }
}  // namespace oft

extern "C" {

int32_t oft_abi_version(void) { return OFT_ABI_VERSION; }

const char* oft_status_str(int32_t s) {
  switch (s) {
    case OFT_OK: return "OFT_OK: success";
    case OFT_EINVAL: return "OFT_EINVAL: null or misaligned pointer, or bad size";
    case OFT_ESHAPE: return "OFT_ESHAPE: shape constraint violated";
    case OFT_EDTYPE: return "OFT_EDTYPE: unknown dtype or weight format";
    case OFT_EUNSUPPORTED: return "OFT_EUNSUPPORTED: configuration not implemented";
    case OFT_EWORKSPACE: return "OFT_EWORKSPACE: workspace too small";
    case OFT_EHIP: return "OFT_EHIP: HIP launch failed (see oft_last_hip_error)";
    default: return "unknown oft status";
  }
}

int32_t oft_last_hip_error(void) { return g_last_hip; }

int32_t cayley_build(const uint16_t* q_bf16, int32_t nblk, int32_t b, float* R_f32,
                     uint16_t* R_ops_or_null, void* stream) {
  if (nblk < 0) return OFT_EINVAL;
  if (b != 16 && b != 32) return OFT_EUNSUPPORTED;
  if (nblk == 0) return OFT_OK;
  if (q_bf16 == nullptr || !ptr_ok(R_f32) || !opt_ok(R_ops_or_null)) return OFT_EINVAL;
  return hip_status(oft::launch_cayley(q_bf16, nblk, b, R_f32, R_ops_or_null,
                                       static_cast<hipStream_t>(stream)));
}

int32_t oft_dequant(int32_t w_fmt, int32_t rows, int32_t cols, int32_t g, const uint8_t* codes,
                    const void* scales, uint16_t* out_bf16, void* stream) {
  if (!w4(w_fmt) && w_fmt != OFT_W_FP8_E4M3) return OFT_EDTYPE;
  if (rows < 0 || cols < 0) return OFT_EINVAL;
  if (cols % 8 != 0) return OFT_ESHAPE;
  if (w4(w_fmt)) {
    if (!group_ok(g)) return OFT_EUNSUPPORTED;
    if (cols % g != 0) return OFT_ESHAPE;
  }
  if ((long long)rows * cols == 0) return OFT_OK;
  if (!ptr_ok(codes) || !ptr_ok(out_bf16)) return OFT_EINVAL;
  if (w4(w_fmt) && !ptr_ok(scales)) return OFT_EINVAL;
  return hip_status(oft::launch_dequant(w_fmt, rows, cols, g, codes, scales, out_bf16,
                                        static_cast<hipStream_t>(stream)));
}

int32_t oft_pack_int4_tiled(int32_t count, int32_t rows, int32_t cols, int32_t g, const uint8_t* codes,
                            const uint16_t* scales, uint8_t* codes_tiled, uint16_t* scales_tiled, void* stream) {
  if (count < 0 || rows < 0 || cols < 0) return OFT_EINVAL;
  if (!group_ok(g)) return OFT_EUNSUPPORTED;
  if (rows % oft::T4_ROWS != 0 || cols % oft::T4_COLS != 0) return OFT_ESHAPE;
  const long long n = (long long)count * rows * cols;
  if (n == 0) return OFT_OK;
  // offsets inside one matrix are 32-bit: rows * cols / 2 code bytes < 2^31
  if ((long long)rows * cols >= (1LL << 32)) return OFT_EUNSUPPORTED;
  if (!ptr_ok(codes) || !ptr_ok(scales) || !ptr_ok(codes_tiled) || !ptr_ok(scales_tiled)) return OFT_EINVAL;
  // the tiled copies may not overlap their sources
  const auto lo = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
  const uintptr_t cb = (uintptr_t)(n / 2), sb = (uintptr_t)(n / g * 2);
  if (lo(codes) < lo(codes_tiled) + cb && lo(codes_tiled) < lo(codes) + cb) return OFT_EINVAL;
  if (lo(scales) < lo(scales_tiled) + sb && lo(scales_tiled) < lo(scales) + sb) return OFT_EINVAL;
  return hip_status(oft::launch_pack_t4(count, rows, cols, g, codes, scales, codes_tiled, scales_tiled,
                                        static_cast<hipStream_t>(stream)));
}

int32_t oft_linear_workspace_bytes(const oft_linear_desc* d, int32_t pass, size_t* bytes) {
  if (bytes == nullptr) return OFT_EINVAL;
  const int32_t v = validate_linear(d);
  if (v != OFT_OK) return v;
  if (pass == OFT_PASS_FWD) {
    *bytes = 0;
  } else if (pass == OFT_PASS_BWD) {
    *bytes = oft::plan_bwd(d->M, d->K, d->N, d->w_fmt == OFT_W_FP8_E4M3, d->w_fmt == OFT_W_INT4,
                       d->x_dtype == OFT_DT_F32).bytes;
  } else {
    return OFT_EINVAL;
  }
  return OFT_OK;
}

int32_t oft_linear_fwd(const oft_linear_desc* d, const void* x, const uint8_t* w_codes,
                       const void* w_scales, const uint16_t* R_ops, void* y, void* ws,
                       size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  const int32_t v = validate_linear(d);
  if (v != OFT_OK) return v;
  if (d->M == 0) return OFT_OK;
  if (!ptr_ok(x) || !ptr_ok(w_codes) || !ptr_ok(w_scales) || !ptr_ok(R_ops) || !ptr_ok(y))
    return OFT_EINVAL;
  return hip_status(oft::launch_linear_fwd(dense_args(d), x, w_codes, w_scales, R_ops, y,
                                           static_cast<hipStream_t>(stream)));
}

int32_t oft_linear_fwd_base(const oft_linear_desc* d, const void* x, const uint8_t* w_codes,
                            const void* w_scales, void* y, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  const int32_t v = validate_linear(d);
  if (v != OFT_OK) return v;
  if (d->M == 0) return OFT_OK;
  if (!ptr_ok(x) || !ptr_ok(w_codes) || !ptr_ok(w_scales) || !ptr_ok(y)) return OFT_EINVAL;
  return hip_status(oft::launch_linear_fwd_base(dense_args(d), x, w_codes, w_scales, y,
                                                static_cast<hipStream_t>(stream)));
}

int32_t oft_slots_switch(int32_t* state, int32_t slot, int32_t version, void* stream) {
  if (!ptr_ok(state) || (slot != 0 && slot != 1)) return OFT_EINVAL;
  return hip_status(oft::launch_slots_switch(state, slot, version, static_cast<hipStream_t>(stream)));
}

int32_t oft_linear_fwd_slots(const oft_linear_desc* d, const void* x, const uint8_t* w_codes,
                             const void* w_scales, const uint16_t* R_ops0, const uint16_t* R_ops1,
                             const int32_t* state, int32_t* latch, void* y, void* ws, size_t ws_bytes,
                             void* stream) {
  (void)ws;
  (void)ws_bytes;
  const int32_t v = validate_linear(d);
  if (v != OFT_OK) return v;
  if (!ptr_ok(state) || !ptr_ok(latch)) return OFT_EINVAL;
  if (d->M > 0 && (!ptr_ok(x) || !ptr_ok(w_codes) || !ptr_ok(w_scales) || !ptr_ok(R_ops0) || !ptr_ok(R_ops1) ||
                   !ptr_ok(y)))
    return OFT_EINVAL;
  return hip_status(oft::launch_linear_fwd_slots(dense_args(d), x, w_codes, w_scales, R_ops0, R_ops1, state, latch,
                                                 y, static_cast<hipStream_t>(stream)));
}

int32_t oft_logprob_diff(int32_t T, int32_t V, const float* logits_actor, const float* logits_ref,
                         const int32_t* labels, float* out, void* stream) {
  if (T < 0 || V < 1 || (long long)T * V >= (1LL << 40)) return OFT_EINVAL;
  if (T == 0) return OFT_OK;
  if (!ptr_ok(logits_actor) || !ptr_ok(logits_ref) || !ptr_ok(labels) || !ptr_ok(out)) return OFT_EINVAL;
  return hip_status(oft::launch_logprob_diff(T, V, logits_actor, logits_ref, labels, out,
                                             static_cast<hipStream_t>(stream)));
}

int32_t oft_linear_bwd(const oft_linear_desc* d, const uint16_t* dy, const void* y_saved,
                       const uint8_t* w_codes, const void* w_scales, const float* R_f32,
                       const uint16_t* R_ops, void* dx_or_null, float* dq_or_null, void* ws,
                       size_t ws_bytes, void* stream) {
  const int32_t v = validate_linear(d);
  if (v != OFT_OK) return v;
  if (!opt_ok(dx_or_null) || !opt_ok(dq_or_null)) return OFT_EINVAL;
  const bool want_dx = dx_or_null != nullptr && d->M > 0;
  const bool want_dq = dq_or_null != nullptr;
  const oft::DqPlan plan = oft::plan_bwd(d->M, d->K, d->N, d->w_fmt == OFT_W_FP8_E4M3, d->w_fmt == OFT_W_INT4,
                       d->x_dtype == OFT_DT_F32);
  if (want_dx) {
    if (!ptr_ok(dy) || !ptr_ok(w_codes) || !ptr_ok(w_scales) || !ptr_ok(R_ops)) return OFT_EINVAL;
  }
  if (want_dq) {
    if (!ptr_ok(R_f32)) return OFT_EINVAL;
    if (d->M > 0 && (!ptr_ok(dy) || !ptr_ok(y_saved))) return OFT_EINVAL;
  }
  if (want_dx || (want_dq && d->M > 0)) {
    if (!ptr_ok(ws)) return OFT_EINVAL;
    if (ws_bytes < plan.bytes) return OFT_EWORKSPACE;
  }
  if (!want_dx && !want_dq) return OFT_OK;
  return hip_status(oft::launch_linear_bwd(dense_args(d), plan, dy, y_saved, w_codes, w_scales, R_f32,
                                           R_ops, want_dx ? dx_or_null : nullptr, dq_or_null,
                                           static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
