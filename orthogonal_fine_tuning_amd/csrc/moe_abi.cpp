// MoE entry points (temporary: not implemented yet).
#include <hip/hip_runtime.h>

#include "oft.h"

extern "C" {

int32_t oft_moe_workspace_bytes(const oft_moe_desc* d, int32_t pass, size_t* bytes) {
  (void)d; (void)pass; (void)bytes;
  return OFT_EUNSUPPORTED;
}

int32_t oft_moe_route(const oft_moe_desc* d, const float* logits, const oft_moe_routing* rt,
                      void* ws, size_t ws_bytes, void* stream) {
  (void)d; (void)logits; (void)rt; (void)ws; (void)ws_bytes; (void)stream;
  return OFT_EUNSUPPORTED;
}

int32_t oft_moe_grouped_fwd(const oft_moe_desc* d, const uint16_t* x, const float* logits,
                            const uint8_t* wgu_codes, const uint16_t* wgu_scales,
                            const uint8_t* wd_codes, const uint16_t* wd_scales,
                            const uint16_t* R_ops, const oft_moe_routing* rt,
                            uint16_t* h_saved, uint16_t* y, void* ws, size_t ws_bytes,
                            void* stream) {
  (void)d; (void)x; (void)logits; (void)wgu_codes; (void)wgu_scales; (void)wd_codes;
  (void)wd_scales; (void)R_ops; (void)rt; (void)h_saved; (void)y; (void)ws; (void)ws_bytes;
  (void)stream;
  return OFT_EUNSUPPORTED;
}

int32_t oft_moe_grouped_bwd(const oft_moe_desc* d, const uint16_t* dy, const oft_moe_routing* rt,
                            const uint16_t* h_saved, const uint8_t* wgu_codes,
                            const uint16_t* wgu_scales, const uint8_t* wd_codes,
                            const uint16_t* wd_scales, const float* R_f32,
                            const uint16_t* R_ops, uint16_t* dx_or_null, float* dq_or_null,
                            float* dw_or_null, void* ws, size_t ws_bytes, void* stream) {
  (void)d; (void)dy; (void)rt; (void)h_saved; (void)wgu_codes; (void)wgu_scales; (void)wd_codes;
  (void)wd_scales; (void)R_f32; (void)R_ops; (void)dx_or_null; (void)dq_or_null;
  (void)dw_or_null; (void)ws; (void)ws_bytes; (void)stream;
  return OFT_EUNSUPPORTED;
}

}  // extern "C"
