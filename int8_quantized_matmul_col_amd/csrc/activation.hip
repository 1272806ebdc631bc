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
// Xq, X_O and W_O are written in the panel-tiled layout of tile_layout.h.
// The mask is kept as bits (ldk/32 words); each block of the row pass
// rebuilds the exclusive prefix count of the mask words in LDS, so a column's
// slot in the compacted slices is prefix[word] + popcount of the lower bits:
// no separate scan launch and no global O list is needed by the consumers.
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

namespace {
constexpr int kColBlock = 512;  // columns per block of the column-absmax pass
constexpr int kRowChunk = kColmaxRowsPerChunk;
}  // namespace

// ---------------------------------------------------------------- column absmax

// grid = ceil(ldk/512) column blocks x ceil(M/64) row chunks (column block
// fastest).  Block 256 = 64 column lanes x 4 row lanes; each lane reads 8
// consecutive columns (16 bytes) of 16 rows of the chunk, all loads issued
// before use.  A wave reads one 1 KiB row segment per load instruction.
__global__ __launch_bounds__(256) void k_colmax_partial(const uint16_t* __restrict__ X, int M,
                                                        int K, int ldk, int vec,
                                                        uint16_t* __restrict__ part) {
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int ncb = (ldk + kColBlock - 1) / kColBlock;
  const int cb = blockIdx.x % ncb, rcix = blockIdx.x / ncb;
  const int c0 = cb * kColBlock + tx * 8;
  const int r0 = rcix * kRowChunk;
  uint32_t mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < K) {
    uint16_t h[16][8];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = r0 + ty + 4 * u;
      if (r < M) {
        load8_half(X + (size_t)r * K, c0, K, vec != 0, h[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) h[u][i] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[i] = max(mx[i], habs_bits(h[u][i]));
  }
  __shared__ uint16_t s[4][kColBlock];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[ty][tx * 8 + i] = (uint16_t)mx[i];
  __syncthreads();
  for (int c = threadIdx.x; c < kColBlock; c += 256) {
    const uint32_t v = max(max((uint32_t)s[0][c], (uint32_t)s[1][c]),
                           max((uint32_t)s[2][c], (uint32_t)s[3][c]));
    const int col = cb * kColBlock + c;
    if (col < ldk) part[(size_t)rcix * ldk + col] = (uint16_t)v;
  }
}

// grid ceil(ldk/64); block 256 = 64 columns x 4 partial lanes.  Reduces the rc
// partials (or, when part == nullptr, the M rows of X directly), compares
// with the threshold and writes the mask bytes (optional) and bit words.
__global__ __launch_bounds__(256) void k_colmask(const uint16_t* __restrict__ X,
                                                 const uint16_t* __restrict__ part, int rc,
                                                 int M, int K, int ldk, float threshold,
                                                 uint8_t* __restrict__ mask8,
                                                 uint32_t* __restrict__ mask_bits) {
  const int cl = threadIdx.x & 63, pl = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cl;
  uint32_t v = 0;
  if (col < K) {
    const int n = part != nullptr ? rc : M;
    int r = pl;
    for (; r + 12 < n; r += 16) {
      uint32_t a0, a1, a2, a3;
      if (part != nullptr) {
        a0 = part[(size_t)r * ldk + col];
        a1 = part[(size_t)(r + 4) * ldk + col];
        a2 = part[(size_t)(r + 8) * ldk + col];
        a3 = part[(size_t)(r + 12) * ldk + col];
      } else {
        a0 = habs_bits(X[(size_t)r * K + col]);
        a1 = habs_bits(X[(size_t)(r + 4) * K + col]);
        a2 = habs_bits(X[(size_t)(r + 8) * K + col]);
        a3 = habs_bits(X[(size_t)(r + 12) * K + col]);
      }
      v = max(v, max(max(a0, a1), max(a2, a3)));
    }
    for (; r < n; r += 4)
      v = max(v, part != nullptr ? (uint32_t)part[(size_t)r * ldk + col]
                                 : habs_bits(X[(size_t)r * K + col]));
  }
  __shared__ uint32_t s[4][64];
  s[pl][cl] = v;
  __syncthreads();
  if (pl == 0) {
    v = max(max(s[0][cl], s[1][cl]), max(s[2][cl], s[3][cl]));
    const bool o = (col < K) && (h2f((uint16_t)v) > threshold);
    if (mask8 != nullptr && col < K) mask8[col] = o ? 1 : 0;
    const uint64_t b = __ballot(o);
    if (cl == 0 && blockIdx.x * 64 < ldk) {
      mask_bits[blockIdx.x * 2] = (uint32_t)b;
      mask_bits[blockIdx.x * 2 + 1] = (uint32_t)(b >> 32);
    }
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

namespace {

// Quantize, store and compact one 8-column chunk c of row m (the chunk's mask
// bits are `word >> sh`).
__device__ __forceinline__ void emit_chunk(const uint16_t h[8], int m, int c, uint32_t word, int sh,
                                           int pre, float a, int ldk, int8_t* __restrict__ Xq,
                                           uint16_t* __restrict__ XO) {
  const uint32_t ob = (word >> sh) & 0xffu;
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int v = quant_code(h2f(h[i]), a);  // computed for every column, then selected
    q[i] = ((ob >> i) & 1u) ? 0 : v;
  }
  uint2 out;
  out.x = (uint32_t)pack4_i8(q[0], q[1], q[2], q[3]);
  out.y = (uint32_t)pack4_i8(q[4], q[5], q[6], q[7]);
  *reinterpret_cast<uint2*>(Xq + tiled_offset(m, (size_t)c * 8, ldk)) = out;
  if (ob && XO != nullptr) {
    int slot = pre + __popc(word & ((1u << sh) - 1u));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((ob >> i) & 1u) {
        XO[tiled_offset(m, (size_t)slot * 2, (size_t)ldk * 2) / 2] = h[i];
        ++slot;
      }
  }
}

}  // namespace

// Row pass.  grid = W_O blocks (16 weight rows each; only when WO !=
// nullptr) followed by row blocks, so the small gather work overlaps the row
// work instead of forming a tail.  WPR = waves per row: 1 (a wave per row, 4
// rows per block) or 4 (the whole block on one row, for few rows).  CPL =
// 8-column chunks per lane held in registers between the absmax and the
// quantize passes (0: re-read the row from L1/L2 instead, for long rows).
// Dynamic LDS: 2*nw words plus the O list (up to kOListCap entries).
constexpr int kOListCap = 4096;
constexpr int kWoRows = 16;

template <int WPR, int CPL>
__global__ __launch_bounds__(256) void k_quant_rows(
    const uint16_t* __restrict__ X, int M, int K, int ldk, int vec, int n_wo_blocks,
    const uint32_t* __restrict__ mask_bits, int8_t* __restrict__ Xq, float* __restrict__ x_scale,
    uint16_t* __restrict__ XO, int32_t* __restrict__ n_out, int32_t* __restrict__ out_idx,
    const int8_t* __restrict__ Wq, const float* __restrict__ w_scale, int N,
    uint16_t* __restrict__ WO) {
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_red[4];
  const int nw = ldk / 32;
  uint32_t* s_bits = s_dyn;
  int* s_pre = reinterpret_cast<int*>(s_dyn + nw);
  const int total = load_mask_prefix(mask_bits, nw, s_bits, s_pre);
  const int opad = (total + 63) & ~63;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int rb = (int)blockIdx.x - n_wo_blocks;  // row block index (< 0: a W_O block)

  if (rb == 0) {
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

  if (rb < 0) {
    // ---- W_O[n][j] for 16 weight rows: the O list in LDS (when it fits),
    // then one (row, j) item per thread and pass, loads issued together.
    int* s_olist = reinterpret_cast<int*>(s_dyn + 2 * nw);
    const bool in_lds = total <= kOListCap;
    if (in_lds) {
      for (int w = t; w < nw; w += 256) {
        uint32_t b = s_bits[w];
        int slot = s_pre[w];
        while (b) {
          s_olist[slot++] = w * 32 + __ffs(b) - 1;
          b &= b - 1;
        }
      }
    }
    __syncthreads();
    const int n0 = blockIdx.x * kWoRows;
    const int nl = t >> 4, jl = t & 15;
    const int n = n0 + nl;
    if (n < N) {
      const float aw = w_scale[n];
      for (int j0 = 0; j0 < opad; j0 += 64) {
        int q[4];
        bool live[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j0 + u * 16 + jl;
          live[u] = j < total;
          q[u] = 0;
          if (live[u]) {
            const int k = in_lds ? s_olist[j] : select_outlier(s_bits, s_pre, nw, j);
            q[u] = (int)Wq[tiled_offset(n, (size_t)k, ldk)];
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j0 + u * 16 + jl;
          WO[tiled_offset(n, (size_t)j * 2, (size_t)ldk * 2) / 2] =
              live[u] ? dequant_w_half(q[u], aw) : (uint16_t)0;
        }
      }
    }
    return;
  }

  // ---- rows
  constexpr int RPB = 4 / WPR;               // rows per block
  constexpr int LPR = 64 * WPR;              // lanes per row
  const int m = rb * RPB + wave / WPR;
  const int rl = (wave % WPR) * 64 + lane;   // lane index within the row
  const int nch = ldk / 8;
  const bool active = m < M;
  const uint16_t* row = X + (size_t)min(m, M - 1) * K;
  uint16_t h[CPL > 0 ? CPL : 1][8];
  uint32_t mx = 0;
  if (CPL > 0) {
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = rl + u * LPR;
      if (c < nch) {
        load8_half(row, c * 8, K, vec != 0, h[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) h[u][i] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = rl + u * LPR;
      const uint32_t ob = c < nch ? (s_bits[c >> 2] >> ((c & 3) * 8)) & 0xffu : 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (!((ob >> i) & 1u)) mx = max(mx, habs_bits(h[u][i]));
    }
  } else {
    for (int c = rl; c < nch; c += LPR) {
      uint16_t g[8];
      load8_half(row, c * 8, K, vec != 0, g);
      const uint32_t ob = (s_bits[c >> 2] >> ((c & 3) * 8)) & 0xffu;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (!((ob >> i) & 1u)) mx = max(mx, habs_bits(g[i]));
    }
  }
  mx = wave_max(mx);
  if (WPR > 1) {
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    mx = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
  }
  const float a = h2f((uint16_t)mx);
  if (active) {
    if (CPL > 0) {
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = rl + u * LPR;
        if (c < nch)
          emit_chunk(h[u], m, c, s_bits[c >> 2], (c & 3) * 8, s_pre[c >> 2], a, ldk, Xq, XO);
      }
    } else {
      for (int c = rl; c < nch; c += LPR) {
        uint16_t g[8];
        load8_half(row, c * 8, K, vec != 0, g);
        emit_chunk(g, m, c, s_bits[c >> 2], (c & 3) * 8, s_pre[c >> 2], a, ldk, Xq, XO);
      }
    }
    if (XO != nullptr)
      for (int j = total + rl; j < opad; j += LPR)
        XO[tiled_offset(m, (size_t)j * 2, (size_t)ldk * 2) / 2] = 0;
    if (rl == 0) x_scale[m] = a;
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
  dim3 grid(((ldk + kColBlock - 1) / kColBlock) * ((M + kRowChunk - 1) / kRowChunk));
  hipLaunchKernelGGL(k_colmax_partial, grid, dim3(256), 0, s, X, M, K, ldk, vec, part);
  return hipGetLastError();
}

hipError_t launch_colmask(const uint16_t* X, const uint16_t* part, int rc, int M, int K,
                          int ldk, float threshold, uint8_t* mask8, uint32_t* mask_bits,
                          hipStream_t s) {
  dim3 grid((ldk + 63) / 64);
  hipLaunchKernelGGL(k_colmask, grid, dim3(256), 0, s, X, part, rc, M, K, ldk, threshold, mask8,
                     mask_bits);
  return hipGetLastError();
}

template <int WPR, int CPL>
static void launch_qr(dim3 grid, size_t lds, hipStream_t s, const uint16_t* X, int M, int K,
                      int ldk, int vec, int nwb, const uint32_t* mb, int8_t* Xq, float* xs,
                      uint16_t* XO, int32_t* n_out, int32_t* out_idx, const int8_t* Wq,
                      const float* ws, int N, uint16_t* WO) {
  hipLaunchKernelGGL((k_quant_rows<WPR, CPL>), grid, dim3(256), lds, s, X, M, K, ldk, vec, nwb, mb,
                     Xq, xs, XO, n_out, out_idx, Wq, ws, N, WO);
}

hipError_t launch_quant_rows(const uint16_t* X, int M, int K, int ldk, const uint32_t* mask_bits,
                             int8_t* Xq, float* x_scale, uint16_t* XO, int32_t* n_out,
                             int32_t* out_idx, const int8_t* Wq, const float* w_scale, int N,
                             uint16_t* WO, hipStream_t s) {
  const int vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  const bool few_rows = M <= 256;  // whole block per row keeps the GPU busy
  const int wpr = few_rows ? 4 : 1;
  const int n_row_blocks = few_rows ? M : (M + 3) / 4;
  const int n_wo_blocks = WO != nullptr ? (N + kWoRows - 1) / kWoRows : 0;
  const size_t lds = (size_t)2 * (ldk / 32) * sizeof(uint32_t) +
                     (WO != nullptr ? (size_t)kOListCap * sizeof(int) : 0);
  dim3 grid(n_row_blocks + n_wo_blocks);
  const int lanes = 64 * wpr;
  const int cpl_needed = (ldk / 8 + lanes - 1) / lanes;
#define QR(W, C) launch_qr<W, C>(grid, lds, s, X, M, K, ldk, vec, n_wo_blocks, mask_bits, Xq, x_scale, XO, n_out, out_idx, Wq, w_scale, N, WO)
  if (wpr == 4) {
    if (cpl_needed <= 4) QR(4, 4);
    else if (cpl_needed <= 8) QR(4, 8);
    else QR(4, 0);
  } else {
    if (cpl_needed <= 2) QR(1, 2);
    else if (cpl_needed <= 4) QR(1, 4);
    else if (cpl_needed <= 8) QR(1, 8);
    else if (cpl_needed <= 16) QR(1, 16);
    else QR(1, 0);
  }
#undef QR
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
