// C ABI of the decomposed int8 matmul (include/int8mm.h): argument checks,
// workspace carving and the launch sequence.  Everything here runs on the
// host; all device work is enqueued on the caller's stream, nothing is
// allocated and the host never waits on the device.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "int8mm.h"
#include "launch.h"
#include "tile_layout.h"

static_assert(INT8MM_MAX_COUNT_THRESHOLDS == i8mm::kMaxCountThresholds,
              "threshold count limit of the header and the kernel");

namespace {

thread_local char g_hip_error[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return INT8MM_EHIP;
}

constexpr size_t kAlign = 256;

// Compute units of the current device (cached per device).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = n;
  }
  return cache[dev];
}
constexpr int64_t kMaxRows = (int64_t)1 << 30;  // M and N: int32 indexing in the kernels

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
int64_t ld_of(int64_t K) { return (K + 63) / 64 * 64; }

// Byte offsets of the workspace regions for one shape.
struct Layout {
  int64_t ldk = 0;
  bool decode = false;
  int rc = 0;  // row chunks of the column-absmax pass (prefill path)
  size_t part = 0, bits = 0, count = 0, xscale = 0, xq = 0, xo = 0, wo = 0, total = 0;
};

Layout make_layout(int64_t M, int64_t K, int64_t N) {
  Layout L;
  L.ldk = ld_of(K);
  L.decode = M <= INT8MM_DECODE_MAX_M;
  L.rc = L.decode ? 0 : (int)((M + i8mm::kColmaxRowsPerChunk - 1) / i8mm::kColmaxRowsPerChunk);
  size_t off = 0;
  L.part = off;   off += align_up((size_t)L.rc * L.ldk * 2);
  L.bits = off;   off += align_up((size_t)(L.ldk / 32) * 4);
  L.count = off;  off += kAlign;
  const size_t Mp = (size_t)i8mm::padded_rows(M), Np = (size_t)i8mm::padded_rows(N);
  L.xscale = off; off += align_up((size_t)M * 4);
  L.xq = off;     off += align_up(Mp * L.ldk);
  L.xo = off;     off += L.decode ? 0 : align_up(Mp * L.ldk * 2);
  L.wo = off;     off += L.decode ? 0 : align_up(Np * L.ldk * 2);
  L.total = off < kAlign ? kAlign : off;
  return L;
}

int check_shape(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0) return INT8MM_ESHAPE;
  if (K > INT8MM_MAX_K || M > kMaxRows || N > kMaxRows) return INT8MM_ESHAPE;
  return INT8MM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
// float16 / float / int32 data: naturally aligned elements
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

struct Outputs {
  uint8_t* mask = nullptr;
  int32_t* n_outliers = nullptr;
  int32_t* outlier_idx = nullptr;
  int8_t* Xq = nullptr;
  float* x_scale = nullptr;
  uint16_t* X_O = nullptr;
  uint16_t* W_O = nullptr;
  int32_t* C = nullptr;
  uint16_t* Y = nullptr;
};

int run(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* w_scale, int64_t N,
        float threshold, const Outputs& out, bool stages, void* ws, size_t ws_bytes,
        hipStream_t s, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
        const uint16_t* bias = nullptr) {
  int st = check_shape(M, K, N);
  if (st != INT8MM_OK) return st;
  if (isnan(threshold) || threshold < 0.0f) return INT8MM_EINVAL;
  if (M == 0 || N == 0) return INT8MM_OK;
  if (!stages && out.Y == nullptr) return INT8MM_EINVAL;
  if (K > 0 && (X == nullptr || Wq == nullptr)) return INT8MM_EINVAL;
  if (w_scale == nullptr) return INT8MM_EINVAL;
  // panel-tiled buffers take 16-byte loads and stores
  if (!aligned16(Wq) || !aligned16(out.Xq) || !aligned16(out.X_O) || !aligned16(out.W_O))
    return INT8MM_EINVAL;
  if (!aligned(X, 2) || !aligned(bias, 2) || !aligned(out.Y, 2) || !aligned(w_scale, 4) ||
      !aligned(out.x_scale, 4) || !aligned(out.C, 4) || !aligned(out.n_outliers, 4) ||
      !aligned(out.outlier_idx, 4))
    return INT8MM_EINVAL;
  const Layout L = make_layout(M, K, N);
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0 || ws_bytes < L.total)
    return INT8MM_EWORKSPACE;

  const int m = (int)M, n = (int)N, k = (int)K, ldk = (int)L.ldk;
  hipError_t e;
  if (K == 0) {
    // Empty contraction: C = 0, no outlier columns, Y = 0.
    // (fill kernels, not hipMemsetAsync: safe inside a captured graph)
    if (out.n_outliers) {
      if ((e = i8mm::launch_zero_half(reinterpret_cast<uint16_t*>(out.n_outliers), 2, s)) != hipSuccess)
        return hip_fail(e);
    }
    if (out.x_scale) {
      if ((e = i8mm::launch_zero_half(reinterpret_cast<uint16_t*>(out.x_scale), 2 * M, s)) != hipSuccess)
        return hip_fail(e);
    }
    if (out.C) {
      if ((e = i8mm::launch_zero_half(reinterpret_cast<uint16_t*>(out.C), 2 * M * N, s)) != hipSuccess)
        return hip_fail(e);
    } else if (out.Y && bias) {
      if ((e = i8mm::launch_bias_rows(bias, M, N, out.Y, s)) != hipSuccess) return hip_fail(e);
    } else if (out.Y) {
      if ((e = i8mm::launch_zero_half(out.Y, M * N, s)) != hipSuccess) return hip_fail(e);
    }
    return INT8MM_OK;
  }

  // Up to four rows with only Y asked for: a single launch that codes X itself.
  const bool stage_out = out.mask || out.n_outliers || out.outlier_idx || out.Xq ||
                         out.x_scale || out.X_O || out.W_O || out.C;
  if (L.decode && !stage_out && out.Y != nullptr && i8mm::gemm_decode_row_ok(X, m, k, ldk, n)) {
    if ((e = i8mm::launch_gemm_decode_row(X, m, k, ldk, threshold, Wq, n, w_scale, bias, out.Y, s,
                                          ev_start, ev_stop)) != hipSuccess)
      return hip_fail(e);
    return INT8MM_OK;
  }

  uint32_t* bits = at<uint32_t>(ws, L.bits);
  int32_t* count = out.n_outliers ? out.n_outliers : at<int32_t>(ws, L.count);
  float* xs = out.x_scale ? out.x_scale : at<float>(ws, L.xscale);
  int8_t* xq = out.Xq ? out.Xq : at<int8_t>(ws, L.xq);
  uint16_t* xo = out.X_O ? out.X_O : (L.decode ? nullptr : at<uint16_t>(ws, L.xo));
  uint16_t* wo = out.W_O ? out.W_O : (L.decode ? nullptr : at<uint16_t>(ws, L.wo));
  // prefill GEMM tiles computed as 256x128 halves (Y output only)
  const int nhalf = !L.decode && out.C == nullptr && out.Y != nullptr
                        ? i8mm::gemm_prefill_nhalf(m, n, device_cus())
                        : 0;

  if (L.decode && i8mm::activation_small_ok(X, m, k, ldk)) {
    // mask and row codes in one launch; the W_O gather (only when asked
    // for) in a launch of its own
    if ((e = i8mm::launch_activation_small(X, m, k, ldk, threshold, out.mask, bits, count,
                                           out.outlier_idx, xq, xs, xo, s)) != hipSuccess)
      return hip_fail(e);
    if (wo != nullptr &&
        (e = i8mm::launch_quant_rows(X, 0, k, ldk, bits, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, Wq, w_scale, n, wo, s)) != hipSuccess)
      return hip_fail(e);
  } else {
    if (L.decode) {
      if ((e = i8mm::launch_colmask(X, nullptr, 0, m, k, ldk, threshold, out.mask, bits, s)) !=
          hipSuccess)
        return hip_fail(e);
    } else {
      uint16_t* part = at<uint16_t>(ws, L.part);
      if ((e = i8mm::launch_colmax_partial(X, m, k, ldk, part, s)) != hipSuccess)
        return hip_fail(e);
      if ((e = i8mm::launch_colmask(X, part, L.rc, m, k, ldk, threshold, out.mask, bits, s)) !=
          hipSuccess)
        return hip_fail(e);
    }
    if ((e = i8mm::launch_quant_rows(X, m, k, ldk, bits, xq, xs, xo, count, out.outlier_idx, Wq,
                                     w_scale, n, wo, s)) != hipSuccess)
      return hip_fail(e);
  }

  uint16_t* Y = out.C ? nullptr : out.Y;
  if (out.C == nullptr && Y == nullptr) return INT8MM_OK;
  if (L.decode)
    e = i8mm::launch_gemm_decode(xq, Wq, m, n, k, ldk, xs, w_scale, X, bits, bias, Y, out.C, s,
                                 ev_start, ev_stop);
  else
    e = i8mm::launch_gemm_prefill(xq, Wq, m, n, k, ldk, xs, w_scale, xo, wo, count, bias, Y,
                                  out.C, nhalf, s, ev_start, ev_stop);
  if (e != hipSuccess) return hip_fail(e);
  return INT8MM_OK;
}

}  // namespace

extern "C" {

INT8MM_API int64_t int8_weight_ld(int64_t K) { return K < 0 ? -1 : ld_of(K); }

INT8MM_API int64_t int8_weight_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K > INT8MM_MAX_K || N > kMaxRows) return -1;
  return i8mm::padded_rows(N) * ld_of(K);
}

INT8MM_API int int8_prepare_weight(const int8mm_half* W, int64_t N, int64_t K, int8_t* Wq, float* w_scale,
                        hipStream_t stream) {
  if (N < 0 || K < 0 || K > INT8MM_MAX_K || N > kMaxRows) return INT8MM_ESHAPE;
  if (N == 0) return INT8MM_OK;
  if (w_scale == nullptr || (K > 0 && (W == nullptr || Wq == nullptr))) return INT8MM_EINVAL;
  if (!aligned16(Wq) || !aligned(W, 2) || !aligned(w_scale, 4)) return INT8MM_EINVAL;
  hipError_t e = i8mm::launch_prepare_weight(W, (int)N, (int)K, (int)ld_of(K), Wq, w_scale, stream);
  if (e != hipSuccess) return hip_fail(e);
  return INT8MM_OK;
}

INT8MM_API int int8_pack_weight(const int8_t* Wq_rowmajor, int64_t N, int64_t K, int8_t* Wq,
                                hipStream_t stream) {
  if (N < 0 || K < 0 || K > INT8MM_MAX_K || N > kMaxRows) return INT8MM_ESHAPE;
  if (N == 0 || K == 0) return INT8MM_OK;
  if (Wq_rowmajor == nullptr || Wq == nullptr) return INT8MM_EINVAL;
  if (!aligned16(Wq)) return INT8MM_EINVAL;
  hipError_t e = i8mm::launch_pack_weight(Wq_rowmajor, (int)N, (int)K, (int)ld_of(K), Wq, stream);
  if (e != hipSuccess) return hip_fail(e);
  return INT8MM_OK;
}

INT8MM_API size_t int8_matmul_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (check_shape(M, K, N) != INT8MM_OK) return 0;
  return make_layout(M, K, N).total;
}

INT8MM_API int int8_matmul(const int8mm_half* X, int64_t M, int64_t K, const int8_t* Wq,
                const float* w_scale, int64_t N, float threshold, int8mm_half* Y,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Outputs out;
  out.Y = Y;
  return run(X, M, K, Wq, w_scale, N, threshold, out, false, workspace, workspace_bytes, stream);
}

INT8MM_API int int8_linear(const int8mm_half* X, int64_t M, int64_t K, const int8_t* Wq,
                           const float* w_scale, int64_t N, const int8mm_half* bias,
                           float threshold, int8mm_half* Y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  Outputs out;
  out.Y = Y;
  return run(X, M, K, Wq, w_scale, N, threshold, out, false, workspace, workspace_bytes, stream,
             nullptr, nullptr, bias);
}

INT8MM_API int int8_column_absmax(const int8mm_half* X, int64_t M, int64_t K,
                                  int8mm_half* colmax, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  int st = check_shape(M, K, 0);
  if (st != INT8MM_OK) return st;
  if (K == 0) return INT8MM_OK;
  if (colmax == nullptr || (M > 0 && X == nullptr)) return INT8MM_EINVAL;
  if (!aligned(X, 2) || !aligned(colmax, 2)) return INT8MM_EINVAL;
  hipError_t e;
  if (M == 0) {  // no rows: every column maximum is 0
    if ((e = i8mm::launch_zero_half(colmax, K, stream)) != hipSuccess) return hip_fail(e);
    return INT8MM_OK;
  }
  const Layout L = make_layout(M, K, 0);
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0 ||
      workspace_bytes < L.total)
    return INT8MM_EWORKSPACE;
  const int m = (int)M, k = (int)K, ldk = (int)L.ldk;
  uint32_t* bits = at<uint32_t>(workspace, L.bits);
  uint16_t* part = nullptr;
  if (!L.decode) {
    part = at<uint16_t>(workspace, L.part);
    if ((e = i8mm::launch_colmax_partial(X, m, k, ldk, part, stream)) != hipSuccess)
      return hip_fail(e);
  }
  if ((e = i8mm::launch_colmask(X, part, L.rc, m, k, ldk, INFINITY, nullptr, bits, stream,
                                colmax)) != hipSuccess)
    return hip_fail(e);
  return INT8MM_OK;
}

INT8MM_API int int8_outlier_counts(const int8mm_half* colmax, int64_t K, const float* thresholds,
                                   int n_thresholds, int32_t* counts, hipStream_t stream) {
  if (K < 0 || K > INT8MM_MAX_K) return INT8MM_ESHAPE;
  if (thresholds == nullptr || counts == nullptr || (K > 0 && colmax == nullptr))
    return INT8MM_EINVAL;
  if (n_thresholds < 1 || n_thresholds > INT8MM_MAX_COUNT_THRESHOLDS) return INT8MM_EINVAL;
  if (!aligned(colmax, 2) || !aligned(counts, 4)) return INT8MM_EINVAL;
  i8mm::CountThresholds thr{};
  for (int i = 0; i < n_thresholds; ++i) {
    if (isnan(thresholds[i]) || thresholds[i] < 0.0f) return INT8MM_EINVAL;
    thr.t[i] = thresholds[i];
  }
  hipError_t e = i8mm::launch_count_above(colmax, (int)K, thr, n_thresholds, counts, stream);
  if (e != hipSuccess) return hip_fail(e);
  return INT8MM_OK;
}

// ---- allocation-free variant of int8_matmul: the workspace is this file's
// static device array, one copy per GPU (held until the process ends).  Host
// code never passes the array's name (a host-side stand-in): its device
// address is looked up once per device and cached.
namespace {

constexpr size_t kScratchBytes = (size_t)INT8MM_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or nullptr with the
// HIP error recorded.
void* scratch_on_current_device(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = hip_fail(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = INT8MM_EINVAL;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *status = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

INT8MM_API int int8_matmul_noalloc(const int8mm_half* X, int64_t M, int64_t K, const int8_t* Wq,
                                   const float* w_scale, int64_t N, float threshold,
                                   int8mm_half* Y, hipStream_t stream) {
  // the size check runs before anything touches the device
  int st = check_shape(M, K, N);
  if (st != INT8MM_OK) return st;
  const size_t need = make_layout(M, K, N).total;
  if (need > kScratchBytes) return INT8MM_ESCRATCH;
  void* ws = scratch_on_current_device(&st);
  if (ws == nullptr) return st;
  Outputs out;
  out.Y = Y;
  return run(X, M, K, Wq, w_scale, N, threshold, out, false, ws, kScratchBytes, stream);
}

INT8MM_API size_t int8_matmul_noalloc_max_workspace(void) { return kScratchBytes; }

INT8MM_API int int8_matmul_profiled(const int8mm_half* X, int64_t M, int64_t K, const int8_t* Wq,
                                    const float* w_scale, int64_t N, float threshold,
                                    int8mm_half* Y, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream, hipEvent_t matmul_start,
                                    hipEvent_t matmul_stop) {
  Outputs out;
  out.Y = Y;
  return run(X, M, K, Wq, w_scale, N, threshold, out, false, workspace, workspace_bytes, stream,
             matmul_start, matmul_stop);
}

INT8MM_API int int8_matmul_stages(const int8mm_half* X, int64_t M, int64_t K, const int8_t* Wq,
                       const float* w_scale, int64_t N, float threshold, uint8_t* mask,
                       int32_t* n_outliers, int32_t* outlier_idx, int8_t* Xq, float* x_scale,
                       int8mm_half* X_O, int8mm_half* W_O, int32_t* C, int8mm_half* Y,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Outputs out;
  out.mask = mask;
  out.n_outliers = n_outliers;
  out.outlier_idx = outlier_idx;
  out.Xq = Xq;
  out.x_scale = x_scale;
  out.X_O = X_O;
  out.W_O = W_O;
  out.C = C;
  out.Y = Y;
  return run(X, M, K, Wq, w_scale, N, threshold, out, true, workspace, workspace_bytes, stream);
}

INT8MM_API const char* int8mm_strerror(int status) {
  switch (status) {
    case INT8MM_OK: return "ok";
    case INT8MM_EINVAL: return "invalid argument (null pointer or bad threshold)";
    case INT8MM_ESHAPE: return "invalid shape (negative dimension or K above the int32 bound)";
    case INT8MM_EWORKSPACE: return "workspace missing, misaligned or too small";
    case INT8MM_EHIP: return "HIP launch failed";
    case INT8MM_ESCRATCH:
      return "shape needs more workspace than int8_matmul_noalloc holds "
             "(int8_matmul_workspace_size > int8_matmul_noalloc_max_workspace)";
    default: return "unknown status";
  }
}

INT8MM_API const char* int8mm_last_hip_error(void) { return g_hip_error; }

}  // extern "C"
