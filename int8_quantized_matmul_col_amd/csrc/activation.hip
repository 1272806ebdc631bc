// Activation pass of the decomposed int8 matmul: outlier-column detection,
// per-row quantization over the regular columns, and compaction of the
// outlier slices.
//
// * Outlier columns: O = { k : max_m |X[m,k]| > t } over the rows of this
//   call ("LLM.int8() notes", section 2.3: the columns whose absolute
//   activation exceeds the threshold, split column-wise from X and row-wise
//   from W).  The comparison is strict.
// * Row quantization: a_x[m] = max over k in R of |X[m,k]|, codes
//   rne(127*x/a_x) in [-127,127] ("PyTorch 2.9 supports LLM.int8()",
//   section 2: dynamic per-input scales, no calibration), 0 in O columns.
// * X_O[m][j] = X[m][O_j]; W_O[n][j] = fp16(fp32(Wq[n][O_j]*a_w[n])/127).
//
// Memory layout: the mask is kept as bits (ldk/32 words); each block of the
// row pass rebuilds the exclusive prefix count of the mask words in LDS, so
// a column's slot in the compacted slices is prefix[word] + popcount of the
// lower bits -- no separate scan launch and no global O list is needed by the
// consumers.
#include "device_common.h"
#include "launch.h"

namespace i8mm {

// ---------------------------------------------------------------- column absmax

// grid ceil(ldk/256) * ceil(M/256) (column block fastest); block 256 = 32 column lanes x 8 row lanes,
// each lane reads 8 consecutive columns (16 bytes) of every 8th row of the
// chunk.  A wave reads 2 rows x 512 contiguous bytes per load.
__global__ __launch_bounds__(256) void k_colmax_partial(const uint16_t* __restrict__ X, int M,
                                                        int K, int ldk, int vec,
                                                        uint16_t* __restrict__ part) {
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int ncb = (ldk + 255) / 256;
  const int cb = blockIdx.x % ncb, rcix = blockIdx.x / ncb;
  const int c0 = cb * 256 + tx * 8;
  const int r0 = rcix * kColmaxRowsPerChunk;
  const int r1 = min(M, r0 + kColmaxRowsPerChunk);
  uint32_t mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < K) {
#pragma unroll 4
    for (int r = r0 + ty; r < r1; r += 8) {
      uint16_t h[8];
      load8_half(X + (size_t)r * K, c0, K, vec != 0, h);
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[i] = max(mx[i], habs_bits(h[i]));
    }
  }
  __shared__ uint16_t s[8][256];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[ty][tx * 8 + i] = (uint16_t)mx[i];
  __syncthreads();
  const int t = threadIdx.x;
  uint32_t v = 0;
#pragma unroll
  for (int y = 0; y < 8; ++y) v = max(v, (uint32_t)s[y][t]);
  const int col = cb * 256 + t;
  if (col < ldk) part[(size_t)rcix * ldk + col] = (uint16_t)v;
}

// grid ceil(ldk/256), one thread per column.  Reduces the rc partials (or, when
// part == nullptr, the M rows of X directly) and compares with the threshold.
// Each wave covers 64 consecutive columns and writes two mask words.
__global__ __launch_bounds__(256) void k_colmask(const uint16_t* __restrict__ X,
                                                 const uint16_t* __restrict__ part, int rc,
                                                 int M, int K, int ldk, float threshold,
                                                 uint8_t* __restrict__ mask8,
                                                 uint32_t* __restrict__ mask_bits) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  uint32_t v = 0;
  if (col < K) {
    if (part != nullptr) {
      for (int r = 0; r < rc; ++r) v = max(v, (uint32_t)part[(size_t)r * ldk + col]);
    } else {
      for (int m = 0; m < M; ++m) v = max(v, habs_bits(X[(size_t)m * K + col]));
    }
  }
  const bool o = (col < K) && (h2f((uint16_t)v) > threshold);
  if (mask8 != nullptr && col < K) mask8[col] = o ? 1 : 0;
  const uint64_t b = __ballot(o);
  const int wave_col0 = col & ~63;
  if ((threadIdx.x & 63) == 0 && wave_col0 < ldk) {
    mask_bits[wave_col0 / 32] = (uint32_t)b;
    mask_bits[wave_col0 / 32 + 1] = (uint32_t)(b >> 32);
  }
}

// ---------------------------------------------------------------- row pass

// Exclusive prefix counts of the mask words into s_pre[], mask words into
// s_bits[]; returns |O|.  Called by all 256 threads of the block.
__device__ int load_mask_prefix(const uint32_t* __restrict__ mask_bits, int nw,
                                uint32_t* s_bits, int* s_pre) {
  __shared__ int s_wsum[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int per = (nw + 255) / 256;
  const int w0 = min(nw, t * per), w1 = min(nw, w0 + per);
  int local = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t b = mask_bits[w];
    s_bits[w] = b;
    local += __popc(b);
  }
  // inclusive scan of `local` across the block
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += (w < wave) ? s_wsum[w] : 0;
    total += s_wsum[w];
  }
  int run = before + incl - local;
  for (int w = w0; w < w1; ++w) {
    s_pre[w] = run;
    run += __popc(s_bits[w]);
  }
  __syncthreads();
  return total;
}

// Column of the j-th outlier (0-based, j < |O|): the last word whose prefix is
// <= j, then the (j - prefix)-th set bit in it.
__device__ __forceinline__ int select_outlier(const uint32_t* s_bits, const int* s_pre, int nw,
                                              int j) {
  int lo = 0, hi = nw - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= j) lo = mid; else hi = mid - 1;
  }
  uint32_t b = s_bits[lo];
  for (int r = j - s_pre[lo]; r > 0; --r) b &= b - 1;
  return lo * 32 + __ffs(b) - 1;
}

// grid = row blocks (rpb rows each, one wave per row) followed by W_O blocks
// (64 weight rows each; only when WO != nullptr).  XO may be nullptr (the
// decode path reads outlier values straight from X).  Dynamic LDS: 2*nw words.
__global__ __launch_bounds__(256) void k_quant_rows(
    const uint16_t* __restrict__ X, int M, int K, int ldk, int vec, int rpb, int n_row_blocks,
    const uint32_t* __restrict__ mask_bits, int8_t* __restrict__ Xq, float* __restrict__ x_scale,
    uint16_t* __restrict__ XO, int32_t* __restrict__ n_out, int32_t* __restrict__ out_idx,
    const int8_t* __restrict__ Wq, const float* __restrict__ w_scale, int N,
    uint16_t* __restrict__ WO) {
  extern __shared__ uint32_t s_dyn[];
  const int nw = ldk / 32;
  uint32_t* s_bits = s_dyn;
  int* s_pre = reinterpret_cast<int*>(s_dyn + nw);
  const int total = load_mask_prefix(mask_bits, nw, s_bits, s_pre);
  const int opad = (total + 63) & ~63;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  if (blockIdx.x == 0) {
    if (t == 0 && n_out != nullptr) *n_out = total;
    if (out_idx != nullptr) {
      for (int w = t; w < nw; w += 256) {
        uint32_t b = s_bits[w];
        int slot = s_pre[w];
        while (b) {
          out_idx[slot++] = w * 32 + __ffs(b) - 1;
          b &= b - 1;
        }
      }
    }
  }

  if ((int)blockIdx.x < n_row_blocks) {
    const int nch = ldk / 8;
    const int m_end = min(M, ((int)blockIdx.x + 1) * rpb);
    for (int m = blockIdx.x * rpb + wave; m < m_end; m += 4) {
      const uint16_t* row = X + (size_t)m * K;
      uint32_t mx = 0;
      for (int c = lane; c < nch; c += 64) {
        uint16_t h[8];
        load8_half(row, c * 8, K, vec != 0, h);
        const uint32_t ob = (s_bits[c >> 2] >> ((c & 3) * 8)) & 0xffu;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (!((ob >> i) & 1u)) mx = max(mx, habs_bits(h[i]));
      }
      mx = wave_max(mx);
      const float a = h2f((uint16_t)mx);
      int8_t* qrow = Xq + (size_t)m * ldk;
      uint16_t* orow = XO != nullptr ? XO + (size_t)m * ldk : nullptr;
      for (int c = lane; c < nch; c += 64) {
        uint16_t h[8];
        load8_half(row, c * 8, K, vec != 0, h);
        const uint32_t word = s_bits[c >> 2];
        const int sh = (c & 3) * 8;
        const uint32_t ob = (word >> sh) & 0xffu;
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = ((ob >> i) & 1u) ? 0 : quant_code(h2f(h[i]), a);
        uint2 out;
        out.x = (uint32_t)pack4_i8(q[0], q[1], q[2], q[3]);
        out.y = (uint32_t)pack4_i8(q[4], q[5], q[6], q[7]);
        *reinterpret_cast<uint2*>(qrow + c * 8) = out;
        if (ob && orow != nullptr) {
          const int base = s_pre[c >> 2] + __popc(word & ((1u << sh) - 1u));
          int r = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if ((ob >> i) & 1u) orow[base + r++] = h[i];
        }
      }
      if (orow != nullptr)
        for (int j = total + lane; j < opad; j += 64) orow[j] = 0;
      if (lane == 0) x_scale[m] = a;
    }
  } else if (WO != nullptr) {
    const int n0 = ((int)blockIdx.x - n_row_blocks) * 64;
    const int items = 64 * opad;
    for (int idx = t; idx < items; idx += 256) {
      const int nl = idx / opad;
      const int j = idx - nl * opad;
      const int n = n0 + nl;
      if (n >= N) break;  // idx grows with nl: every later item is past N too
      uint16_t v = 0;
      if (j < total) {
        const int k = select_outlier(s_bits, s_pre, nw, j);
        v = dequant_w_half((int)Wq[(size_t)n * ldk + k], w_scale[n]);
      }
      WO[(size_t)n * ldk + j] = v;
    }
  }
}

__global__ void k_zero_half(uint16_t* __restrict__ Y, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    Y[i] = 0;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_colmax_partial(const uint16_t* X, int M, int K, int ldk, uint16_t* part,
                                 hipStream_t s) {
  const int vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  dim3 grid(((ldk + 255) / 256) * ((M + kColmaxRowsPerChunk - 1) / kColmaxRowsPerChunk));
  hipLaunchKernelGGL(k_colmax_partial, grid, dim3(256), 0, s, X, M, K, ldk, vec, part);
  return hipGetLastError();
}

hipError_t launch_colmask(const uint16_t* X, const uint16_t* part, int rc, int M, int K,
                          int ldk, float threshold, uint8_t* mask8, uint32_t* mask_bits,
                          hipStream_t s) {
  dim3 grid((ldk + 255) / 256);
  hipLaunchKernelGGL(k_colmask, grid, dim3(256), 0, s, X, part, rc, M, K, ldk, threshold, mask8,
                     mask_bits);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* X, int M, int K, int ldk, const uint32_t* mask_bits,
                             int8_t* Xq, float* x_scale, uint16_t* XO, int32_t* n_out,
                             int32_t* out_idx, const int8_t* Wq, const float* w_scale, int N,
                             uint16_t* WO, hipStream_t s) {
  const int vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  int rpb = (M + 511) / 512;
  rpb = ((rpb + 3) / 4) * 4;
  if (rpb < 4) rpb = 4;
  if (rpb > 32) rpb = 32;
  const int n_row_blocks = (M + rpb - 1) / rpb;
  const int n_wo_blocks = WO != nullptr ? (N + 63) / 64 : 0;
  const size_t lds = (size_t)2 * (ldk / 32) * sizeof(uint32_t);
  dim3 grid(n_row_blocks + n_wo_blocks);
  hipLaunchKernelGGL(k_quant_rows, grid, dim3(256), lds, s, X, M, K, ldk, vec, rpb, n_row_blocks,
                     mask_bits, Xq, x_scale, XO, n_out, out_idx, Wq, w_scale, N, WO);
  return hipGetLastError();
}

hipError_t launch_zero_half(uint16_t* Y, int64_t count, hipStream_t s) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_zero_half, dim3((unsigned)blocks), dim3(256), 0, s, Y, count);
  return hipGetLastError();
}

}  // namespace i8mm
