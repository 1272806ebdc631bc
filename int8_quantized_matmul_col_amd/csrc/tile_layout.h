// Panel-tiled operand layout shared by the kernels that write and read the
// int8 operands (Xq, the prepared Wq) and the fp16 outlier slices (X_O, W_O).
//
// A matrix of R rows, each `row_bytes` long (a multiple of 64), is stored as
// panels of 256 rows; inside a panel, 64-byte column blocks follow each
// other, and one block holds its 256 row pieces back to back:
//
//   offset(r, b) = ((r / 256) * (row_bytes / 64) + b / 64) * 16384
//                + (r % 256) * 64 + b % 64
//
// so one 64-byte K step of a 256-row panel is 16 KiB of contiguous memory:
// the GEMM's wave loads read whole cache lines (a row-major layout would
// give 16 half lines per wave load instruction, half the L2->CU throughput
// on gfx950), and a 16-row group of the decode kernel is 1 KiB contiguous.
// Rows are padded to a multiple of 256 (padded_rows).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace i8mm {

constexpr int kPanelRows = 256;
constexpr int kTileK = 64;                        // bytes of a column block
constexpr int kTileBytes = kPanelRows * kTileK;  // 16 KiB

__host__ __device__ inline size_t tiled_offset(int r, size_t b, size_t row_bytes) {
  return ((size_t)(r >> 8) * (row_bytes >> 6) + (b >> 6)) * (size_t)kTileBytes +
         (size_t)(r & 255) * 64 + (b & 63);
}

__host__ __device__ inline int64_t padded_rows(int64_t R) {
  return (R + kPanelRows - 1) / kPanelRows * kPanelRows;
}

}  // namespace i8mm
