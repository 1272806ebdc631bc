// Host-side launchers of the gfx950 kernels (internal to the library; the
// public C ABI is include/int8mm.h).  Each returns the HIP status of its
// launch.  Shapes are validated by the caller (api.hip) before any launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

// Rows of X reduced by one block of the column-absmax pass (prefill path).
constexpr int kColmaxRowsPerChunk = 64;

hipError_t launch_prepare_weight(const uint16_t* W, int N, int K, int ldk, int8_t* Wq,
                                 float* w_scale, hipStream_t s);
// Row-major int8 codes [N][K] into the panel-tiled layout (clamped to +-127,
// zero padding).
hipError_t launch_pack_weight(const int8_t* src, int N, int K, int ldk, int8_t* Wq,
                              hipStream_t s);

// Prefill: per-chunk column absmax partials part[rc][ldk] (u16 |x| bits).
hipError_t launch_colmax_partial(const uint16_t* X, int M, int K, int ldk, uint16_t* part,
                                 hipStream_t s);
// Reduces the partials (rc > 0) or scans X directly (part == nullptr, small
// M) into the outlier mask: bytes mask8[K] (optional) and bits mask_bits[ldk/32];
// optionally the column maxima themselves, colmax[K] (|x| binary16 bits).
hipError_t launch_colmask(const uint16_t* X, const uint16_t* part, int rc, int M, int K,
                          int ldk, float threshold, uint8_t* mask8, uint32_t* mask_bits,
                          hipStream_t s, uint16_t* colmax = nullptr);
// Row quantization over R, outlier compaction, |O| and the O list; optionally
// the dequantized outlier weight rows W_O (when WO != nullptr).
hipError_t launch_quant_rows(const uint16_t* X, int M, int K, int ldk, const uint32_t* mask_bits,
                             int8_t* Xq, float* x_scale, uint16_t* XO, int32_t* n_out,
                             int32_t* out_idx, const int8_t* Wq, const float* w_scale, int N,
                             uint16_t* WO, hipStream_t s);
// Prefill tile GEMM: int8 MFMA over K, then fp16 MFMA over the outlier slice,
// fused dequant epilogue (Y, plus bias[n] when bias != nullptr), or int32
// accumulators only (C).
// nhalf (Y only; 0 .. tile count, else hipErrorInvalidValue): the last nhalf
// tiles are computed as two 256x128 halves each.
hipError_t launch_gemm_prefill(const int8_t* Xq, const int8_t* Wq, int M, int N, int K, int ldk,
                               const float* x_scale, const float* w_scale, const uint16_t* XO,
                               const uint16_t* WO, const int32_t* n_out, const uint16_t* bias,
                               uint16_t* Y, int32_t* C, int nhalf, hipStream_t s,
                               hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// How many tiles the GEMM computes as halves for this shape on a GPU of n_cu
// CUs.
int gemm_prefill_nhalf(int M, int N, int n_cu);
// e0/e1 (optional) are stamped by the GEMM dispatch itself: start and end of
// that kernel, for profiling.
// Decode (M <= 16): one streaming pass over Wq, outliers handled inline.
hipError_t launch_gemm_decode(const int8_t* Xq, const int8_t* Wq, int M, int N, int K, int ldk,
                              const float* x_scale, const float* w_scale, const uint16_t* X,
                              const uint32_t* mask_bits, const uint16_t* bias, uint16_t* Y,
                              int32_t* C, hipStream_t s, hipEvent_t e0 = nullptr,
                              hipEvent_t e1 = nullptr);
// One to four rows, Y output: the same kernel deriving the mask, a_x and the
// codes of X itself, so the call is a single launch.  Applicable when
// gemm_decode_row_ok() (M <= 4, K % 8 == 0, X 16-byte aligned, ldk <= 16384
// for one row, <= 8192 and N <= 28672 for two to four).
bool gemm_decode_row_ok(const uint16_t* X, int M, int K, int ldk, int N);
hipError_t launch_gemm_decode_row(const uint16_t* X, int M, int K, int ldk, float threshold,
                                  const int8_t* Wq, int N, const float* w_scale,
                                  const uint16_t* bias, uint16_t* Y, hipStream_t s,
                                  hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// Y[0 .. count) = 0 (K == 0 case).
hipError_t launch_zero_half(uint16_t* Y, int64_t count, hipStream_t s);
// Thresholds of one int8_outlier_counts call, passed by value (kernel
// arguments): at most kMaxCountThresholds of them.
constexpr int kMaxCountThresholds = 64;
struct CountThresholds {
  float t[kMaxCountThresholds];
};
hipError_t launch_count_above(const uint16_t* colmax, int K, const CountThresholds& thr, int n,
                              int32_t* counts, hipStream_t s);
// Y[m][n] = bias[n] for an [M][N] Y (K == 0 case with a bias).
hipError_t launch_bias_rows(const uint16_t* bias, int64_t M, int64_t N, uint16_t* Y,
                            hipStream_t s);
// Few rows (M <= 16): mask and row quantization in one launch (grid = M).
// Applicable when activation_small_ok(); X_O optional, no W_O.
bool activation_small_ok(const uint16_t* X, int M, int K, int ldk);
hipError_t launch_activation_small(const uint16_t* X, int M, int K, int ldk, float threshold,
                                   uint8_t* mask8, uint32_t* mask_bits, int32_t* n_out,
                                   int32_t* out_idx, int8_t* Xq, float* x_scale, uint16_t* XO,
                                   hipStream_t s);

}  // namespace i8mm
