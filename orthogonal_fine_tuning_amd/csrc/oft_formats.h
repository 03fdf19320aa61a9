// Weight formats of the GEMM kernels (host and device code).
#pragma once

#include <cstdint>

namespace oft {

// INT4 codes + fp16 group scales, FP8 e4m3 codes (scale per output channel,
// applied outside the K loop), bf16 values (already dequantised), FP4 (OCP
// MX E2M1 codes + E8M0 group exponents, laid out as INT4), or INT4 stored in
// tiles (WF_INT4T: the INT4 values, codes and scales permuted as below)
enum : int { WF_INT4 = 0, WF_FP8 = 1, WF_BF16 = 2, WF_FP4 = 3, WF_INT4T = 4 };

// the 4-bit formats: codes two per byte, low nibble first, and one 16-bit
// scale slot per group of g codes along K (row-major, or tiled for WF_INT4T)
constexpr bool wf_4bit(int wf) { return wf == WF_INT4 || wf == WF_FP4 || wf == WF_INT4T; }
constexpr bool wf_tiled(int wf) { return wf == WF_INT4T; }

// Tiled 4-bit storage of an [N, K] weight (N % 64 == 0, K % 128 == 0): tiles
// of 64 rows x 128 columns, tile (rb, kb) the (rb * K/128 + kb)-th.
//   codes   4096 bytes a tile, row r of the tile at byte 64 r (its 128 codes
//           as in a row-major row: two per byte, low nibble first)
//   scales  64 x 128/g slots a tile (16384/g bytes), row r at byte r 256/g
//           (its 128/g slots in column order)
// so one weight row's codes for 128 consecutive columns are 64 contiguous
// bytes, a tile's 64 rows of them are 4 KB contiguous, and the scales that
// go with them follow the same order.
constexpr int T4_ROWS = 64, T4_COLS = 128, T4_TILE_BYTES = 4096;
// byte offset of code byte `byte` (columns 2 byte, 2 byte + 1) of row `row`
__host__ __device__ constexpr uint32_t t4_code_off(int row, int byte, int K) {
  return (uint32_t)(((row >> 6) * (K >> 7) + (byte >> 6)) * T4_TILE_BYTES + (row & 63) * 64 + (byte & 63));
}
// byte offset of scale slot j (columns [j g, j g + g)) of row `row`
__host__ __device__ constexpr uint32_t t4_scale_off(int row, int j, int K, int g) {
  return (uint32_t)(((row >> 6) * (K >> 7) + ((j * g) >> 7)) * (16384 / g) + (row & 63) * (256 / g) +
                    2 * (j % (128 / g)));
}

}  // namespace oft
