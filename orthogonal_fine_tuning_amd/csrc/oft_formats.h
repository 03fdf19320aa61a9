// Weight formats of the GEMM kernels (host and device code).
#pragma once

namespace oft {

// INT4 codes + fp16 group scales, FP8 e4m3 codes (scale per output channel,
// applied outside the K loop), or bf16 values (already dequantised)
enum : int { WF_INT4 = 0, WF_FP8 = 1, WF_BF16 = 2 };

}  // namespace oft
