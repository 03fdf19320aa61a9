// Weight formats of the GEMM kernels (host and device code).
#pragma once

namespace oft {

// INT4 codes + fp16 group scales, FP8 e4m3 codes (scale per output channel,
// applied outside the K loop), bf16 values (already dequantised), or FP4
// (OCP MX E2M1 codes + E8M0 group exponents, laid out as INT4)
enum : int { WF_INT4 = 0, WF_FP8 = 1, WF_BF16 = 2, WF_FP4 = 3 };

// the two 4-bit formats share every layout: codes two per byte, low nibble
// first, and one 16-bit scale slot per group of g codes
constexpr bool wf_4bit(int wf) { return wf == WF_INT4 || wf == WF_FP4; }

}  // namespace oft
