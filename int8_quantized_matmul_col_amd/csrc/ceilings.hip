// Measurement probes (not part of the matmul path): the practical ceilings
// that the matmul kernels are set against, measured on the GPU at hand.
//
//  * int8 MFMA issue rate: every wave keeps 16 independent
//    v_mfma_i32_32x32x32_i8 accumulators busy on operands loaded once from a
//    caller buffer (random bytes, or zeros), one workgroup of 4 waves per
//    SIMD quad, a grid of `blocks` workgroups.  The rate depends on the data:
//    the chip's clock under MFMA load is power-limited.
//  * HBM read rate: each workgroup streams a contiguous chunk of the buffer
//    with 8 independent 16-byte loads per lane in flight (the fastest of the
//    load shapes tried), folding the data into one word per lane so nothing
//    is skipped.
//
// Built into a library of its own (libint8mm_ceilings.so) that only the
// benchmark loads.  Each entry point runs its warm-up and timed launches on
// the null stream, synchronizes, and returns hipSuccess or the first error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_mfma_i8(const v4i* __restrict__ src, int iters,
                                                 int* __restrict__ out) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  v4i a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = src[(t * 8 + 2 * i) & 4095];
    b[i] = src[(t * 8 + 2 * i + 1) & 4095];
  }
  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j], a[i], acc[i][j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[t] = s;
}

constexpr int kReadU = 8;

// Workgroup b reads vectors [b*per, (b+1)*per) of src, per = n / gridDim.x
// (a multiple of 256 * kReadU, checked by the host).
__global__ __launch_bounds__(256) void k_read_chunk(const v4i* __restrict__ src, size_t per,
                                                    int* __restrict__ out) {
  const v4i* p = src + (size_t)blockIdx.x * per;
  v4i s = {0, 0, 0, 0};
  for (size_t i = threadIdx.x; i < per; i += 256 * kReadU) {
    v4i v[kReadU];
#pragma unroll
    for (int u = 0; u < kReadU; ++u) v[u] = p[i + u * 256];
#pragma unroll
    for (int u = 0; u < kReadU; ++u) s ^= v[u];
  }
  out[blockIdx.x * 256 + threadIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

template <typename F>
hipError_t timed(F launch, int reps, float* ms) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  for (int w = 0; w < 3 && e == hipSuccess; ++w) {
    launch();
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipEventRecord(e0, nullptr);
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    launch();
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return e;
}

}  // namespace

extern "C" {

// int8 MFMA rate in ops/s (2 per multiply-add) into *ops_per_s.  src: 64 KiB
// of operand bytes (device), out: blocks*256 ints (device).
__attribute__((visibility("default"))) int int8mm_probe_mfma_i8(const void* src, int blocks,
                                                                int iters, int* out,
                                                                double* ops_per_s) {
  if (src == nullptr || out == nullptr || ops_per_s == nullptr || blocks <= 0 || iters <= 0)
    return (int)hipErrorInvalidValue;
  float ms = 0.0f;
  const int reps = 10;
  hipError_t e = timed(
      [&] {
        hipLaunchKernelGGL(k_mfma_i8, dim3(blocks), dim3(256), 0, nullptr,
                           static_cast<const v4i*>(src), iters, out);
      },
      reps, &ms);
  if (e != hipSuccess) return (int)e;
  // per wave and iteration: 16 MFMAs of 32x32x32 multiply-adds
  const double ops = (double)reps * blocks * 4 * (double)iters * 16 * 32768.0 * 2.0;
  *ops_per_s = ops / (ms * 1e-3);
  return 0;
}

// HBM read rate in bytes/s into *bytes_per_s over `bytes` of src (device).
// bytes must be a multiple of blocks * 256 * 8 * 16; out: blocks*256 ints.
__attribute__((visibility("default"))) int int8mm_probe_read(const void* src, size_t bytes,
                                                             int blocks, int* out,
                                                             double* bytes_per_s) {
  const size_t unit = (size_t)blocks * 256 * kReadU * 16;
  if (src == nullptr || out == nullptr || bytes_per_s == nullptr || blocks <= 0 ||
      bytes == 0 || bytes % unit != 0)
    return (int)hipErrorInvalidValue;
  const size_t per = bytes / 16 / (size_t)blocks;
  float ms = 0.0f;
  const int reps = 5;
  hipError_t e = timed(
      [&] {
        hipLaunchKernelGGL(k_read_chunk, dim3(blocks), dim3(256), 0, nullptr,
                           static_cast<const v4i*>(src), per, out);
      },
      reps, &ms);
  if (e != hipSuccess) return (int)e;
  *bytes_per_s = (double)reps * bytes / (ms * 1e-3);
  return 0;
}

// The same stream over `copies` buffers of `bytes` each (src, src + bytes,
// ...), launch r reading copy r % copies: with copies * bytes beyond the
// 256 MB MALL every launch reads from HBM, and a buffer the size of one call's
// operand gives the rate of back-to-back launches of that size (ramp and
// tail included).  bytes must be a multiple of blocks * 256 * 8 * 16.
__attribute__((visibility("default"))) int int8mm_probe_read_copies(const void* src,
                                                                    size_t bytes, int copies,
                                                                    int blocks, int* out,
                                                                    double* bytes_per_s) {
  const size_t unit = (size_t)blocks * 256 * kReadU * 16;
  if (src == nullptr || out == nullptr || bytes_per_s == nullptr || blocks <= 0 ||
      copies <= 0 || bytes == 0 || bytes % unit != 0)
    return (int)hipErrorInvalidValue;
  const size_t per = bytes / 16 / (size_t)blocks;
  float ms = 0.0f;
  const int reps = 5 * copies;
  int r = 0;
  hipError_t e = timed(
      [&] {
        const v4i* c = static_cast<const v4i*>(src) + (size_t)(r++ % copies) * (bytes / 16);
        hipLaunchKernelGGL(k_read_chunk, dim3(blocks), dim3(256), 0, nullptr, c, per, out);
      },
      reps, &ms);
  if (e != hipSuccess) return (int)e;
  *bytes_per_s = (double)reps * bytes / (ms * 1e-3);
  return 0;
}

}  // extern "C"
