// oft_linear_bwd_noalloc (include/oft.h): the dense backward on a fixed
// device scratch array instead of a caller workspace, for callers that must
// not allocate (code under graph capture, tight serving loops).
//
// The array is a file-scope device variable of OFT_NOALLOC_SCRATCH_BYTES,
// held by every GPU the library runs on until the process ends.  Host code
// never uses its name as an address: on the first call on each device (that
// device current) hipGetSymbolAddress gives that device's copy, kept per
// device, and the launches take that pointer exactly as they take the
// workspace of oft_linear_bwd.  The kernels write every scratch byte they
// read (partial sums, the rotated gradient, the transposed weight), so no
// part of it needs clearing between calls; calls that overlap on one GPU
// share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "oft.h"
#include "oft_launch.h"

static __device__ __align__(256) unsigned char scratch[OFT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAXDEV = 64;
std::mutex g_mu;
void* g_ptr[MAXDEV] = {};

// this device's copy of the scratch array, looked up once per device
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int32_t oft_linear_bwd_noalloc(const oft_linear_desc* d, const uint16_t* dy, const void* y_saved,
                                          const uint8_t* w_codes, const void* w_scales, const float* R_f32,
                                          const uint16_t* R_ops, void* dx_or_null, float* dq_or_null,
                                          void* stream) {
  size_t need = 0;
  const int32_t v = oft_linear_workspace_bytes(d, OFT_PASS_BWD, &need);  // validates the descriptor
  if (v != OFT_OK) return v;
  if (need > OFT_NOALLOC_SCRATCH_BYTES) return OFT_EWORKSPACE;
  const bool want_dx = dx_or_null != nullptr && d->M > 0;
  const bool want_dq = dq_or_null != nullptr;
  if (!want_dx && !want_dq) {
    // nothing the scratch would serve: the plain call's own checks and no-op
    return oft_linear_bwd(d, dy, y_saved, w_codes, w_scales, R_f32, R_ops, dx_or_null, dq_or_null, nullptr, 0,
                          stream);
  }
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) {
    oft::set_last_hip_error(static_cast<int>(e));
    return OFT_EHIP;
  }
  return oft_linear_bwd(d, dy, y_saved, w_codes, w_scales, R_f32, R_ops, dx_or_null, dq_or_null, ws,
                        OFT_NOALLOC_SCRATCH_BYTES, stream);
}
