// One-time per-output-channel weight quantization ("PyTorch 2.9 supports
// LLM.int8()", section 1: one absmax/127 scale per output channel, weights
// rounded to int8 once, before the first inference).
//
// One wave per weight row: pass 1 reduces max |W[n,:]| with 16-byte loads and
// a wave max, pass 2 re-reads the row (L1/L2 hit) and writes the int8 codes
// 8 at a time into the panel-tiled layout (tile_layout.h), zero-padded to
// ldk columns and to a multiple of 256 rows.
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

__global__ __launch_bounds__(256) void k_prepare_weight(const uint16_t* __restrict__ W, int N,
                                                        int K, int ldk, int vec,
                                                        int8_t* __restrict__ Wq,
                                                        float* __restrict__ w_scale) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = ldk / 8;
  if (n >= N) {  // padding rows of the last panel: zeros
    for (int c = lane; c < nch; c += 64)
      *reinterpret_cast<uint2*>(Wq + tiled_offset(n, (size_t)c * 8, ldk)) = uint2{0u, 0u};
    return;
  }
  const uint16_t* row = W + (size_t)n * K;
  uint32_t mx = 0;
  for (int c = lane; c < nch; c += 64) {
    uint16_t h[8];
    load8_half(row, c * 8, K, vec != 0, h);
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = max(mx, habs_bits(h[i]));
  }
  mx = wave_max(mx);
  const float a = h2f((uint16_t)mx);
  for (int c = lane; c < nch; c += 64) {
    uint16_t h[8];
    load8_half(row, c * 8, K, vec != 0, h);
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quant_code(h2f(h[i]), a);  // pad columns hold 0 -> code 0
    uint2 out;
    out.x = (uint32_t)pack4_i8(q[0], q[1], q[2], q[3]);
    out.y = (uint32_t)pack4_i8(q[4], q[5], q[6], q[7]);
    *reinterpret_cast<uint2*>(Wq + tiled_offset(n, (size_t)c * 8, ldk)) = out;
  }
  if (lane == 0) w_scale[n] = a;
}

hipError_t launch_prepare_weight(const uint16_t* W, int N, int K, int ldk, int8_t* Wq,
                                 float* w_scale, hipStream_t s) {
  const int vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
  dim3 grid((unsigned)(padded_rows(N) / 4));
  hipLaunchKernelGGL(k_prepare_weight, grid, dim3(256), 0, s, W, N, K, ldk, vec, Wq, w_scale);
  return hipGetLastError();
}

}  // namespace i8mm
