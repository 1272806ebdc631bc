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
// For a few rows (M <= 16) k_activation_small does the mask and the codes in
// one launch.
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

namespace {
constexpr int kColBlock = 512;  // columns per block of the column-absmax pass
constexpr int kRowChunk = kColmaxRowsPerChunk;
}  // namespace

// ---------------------------------------------------------------- column absmax

// grid = ceil(ldk/512) column blocks x ceil(M/kRowChunk) row chunks.  Workgroups
// go round-robin to the 8 XCDs; when the chunk count is a multiple of 8,
// chunk c is read only by workgroups on XCD c % 8 (each XCD reads whole rows,
// the same rows the row pass reads there); otherwise column block fastest.
// Block 256 = 64 column lanes x 4 row lanes; each lane reads 8
// consecutive columns (16 bytes) of kRowChunk/4 rows of the chunk, all loads issued
// before use.  A wave reads one 1 KiB row segment per load instruction.
__global__ __launch_bounds__(256) void k_colmax_partial(const uint16_t* __restrict__ X, int M,
                                                        int K, int ldk, int vec,
                                                        uint16_t* __restrict__ part) {
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int ncb = (ldk + kColBlock - 1) / kColBlock;
  const int rcn = (int)gridDim.x / ncb;
  int cb, rcix;
  if (rcn % 8 == 0) {
    const int x = blockIdx.x & 7, q = blockIdx.x >> 3;
    rcix = 8 * (q / ncb) + x;
    cb = q % ncb;
  } else {
    cb = blockIdx.x % ncb;
    rcix = blockIdx.x / ncb;
  }
  const int c0 = cb * kColBlock + tx * 8;
  const int r0 = rcix * kRowChunk;
  uint32_t mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < K) {
    constexpr int kU = kRowChunk / 4;  // rows per lane
    uint16_t h[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = r0 + ty + 4 * u;
      if (r < M) {
        load8_half(X + (size_t)r * K, c0, K, vec != 0, h[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) h[u][i] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
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
                                                 uint32_t* __restrict__ mask_bits,
                                                 uint16_t* __restrict__ colmax) {
  const int cl = threadIdx.x & 63, pl = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cl;
  uint32_t v = 0;
  if (col < K) {
    // 16 independent loads per lane and round (one round for rc <= 64)
    constexpr int kU = 16;
    if (part != nullptr) {
      for (int r0 = pl; r0 < rc; r0 += 4 * kU) {
        uint32_t a[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int r = r0 + 4 * u;
          a[u] = r < rc ? (uint32_t)part[(size_t)r * ldk + col] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) v = max(v, a[u]);
      }
    } else {
      for (int r0 = pl; r0 < M; r0 += 4 * kU) {
        uint32_t a[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int r = r0 + 4 * u;
          a[u] = r < M ? habs_bits(X[(size_t)r * K + col]) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) v = max(v, a[u]);
      }
    }
  }
  __shared__ uint32_t s[4][64];
  s[pl][cl] = v;
  __syncthreads();
  if (pl == 0) {
    v = max(max(s[0][cl], s[1][cl]), max(s[2][cl], s[3][cl]));
    const bool o = (col < K) && (h2f((uint16_t)v) > threshold);
    if (mask8 != nullptr && col < K) mask8[col] = o ? 1 : 0;
    if (colmax != nullptr && col < K) colmax[col] = (uint16_t)v;
    const uint64_t b = __ballot(o);
    if (cl == 0 && blockIdx.x * 64 < ldk) {
      mask_bits[blockIdx.x * 2] = (uint32_t)b;
      mask_bits[blockIdx.x * 2 + 1] = (uint32_t)(b >> 32);
    }
  }
}

// ---------------------------------------------------------------- row pass

// Exclusive prefix counts of the mask words into s_pre[], mask words into
// s_bits[] (from mask_bits; or already there when mask_bits is null); returns
// |O|.  Called by all T threads of the block.
template <int T = 256>
__device__ int load_mask_prefix(const uint32_t* __restrict__ mask_bits, int nw,
                                uint32_t* s_bits, int* s_pre) {
  __shared__ int s_wsum[T / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int per = (nw + T - 1) / T;
  const int w0 = min(nw, t * per), w1 = min(nw, w0 + per);
  int local = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t b;
    if (mask_bits != nullptr) {
      b = mask_bits[w];
      s_bits[w] = b;
    } else {
      b = s_bits[w];
    }
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
  for (int w = 0; w < T / 64; ++w) {
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

// The same prefix for mask words already in s_bits[], computed by wave 0
// alone (each lane a run of consecutive words, one wave scan) and |O| handed
// to every thread through LDS: one barrier, no cross-wave sums.  For the
// 1024-thread single-launch decode pass, where the block-wide scan's
// barriers and per-wave sums cost about a microsecond.
template <int T>
__device__ int mask_prefix_wave0(int nw, const uint32_t* s_bits, int* s_pre) {
  __shared__ int s_total;
  const int t = threadIdx.x, lane = t & 63;
  if (t < 64) {
    const int per = (nw + 63) / 64;
    const int w0 = min(nw, lane * per), w1 = min(nw, w0 + per);
    int local = 0;
    for (int w = w0; w < w1; ++w) local += __popc(s_bits[w]);
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    int run = incl - local;
    for (int w = w0; w < w1; ++w) {
      s_pre[w] = run;
      run += __popc(s_bits[w]);
    }
    if (lane == 63) s_total = incl;
  }
  __syncthreads();
  return s_total;
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

// Outlier columns of one chunk of row m (mask bits ob = (word >> sh) & 0xff,
// ob != 0): their codes zeroed, their values copied to the outlier slice at
// slots pre + (set bits of word below sh), ...
__device__ __forceinline__ void outlier_chunk(uint2& q, const uint4& w, int m, uint32_t word,
                                              int sh, int pre, int ldk,
                                              uint16_t* __restrict__ XO) {
  const uint32_t ob = (word >> sh) & 0xffu;
  q.x &= keep_bytes(ob & 0xfu);
  q.y &= keep_bytes(ob >> 4);
  if (XO != nullptr) {
    int slot = pre + __popc(word & ((1u << sh) - 1u));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((ob >> i) & 1u) {
        XO[tiled_offset(m, (size_t)slot * 2, (size_t)ldk * 2) / 2] = (uint16_t)half_at(w, i);
        ++slot;
      }
  }
}

// Codes of one chunk with both fix-ups (the form used when a row is streamed
// chunk by chunk).
__device__ __forceinline__ uint2 code_chunk(const uint4& w, int m, uint32_t word, int sh, int pre,
                                            float r, float a, int ldk,
                                            uint16_t* __restrict__ XO) {
  float dev;
  uint2 q = quant8_fast(w, r, &dev);
  if (dev > kTieGuard) q = quant8_exact(w, a);
  if ((word >> sh) & 0xffu) outlier_chunk(q, w, m, word, sh, pre, ldk, XO);
  return q;
}

// s_waitcnt vmcnt(0), other counters left alone.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

}  // namespace

// Chunks rl, rl + LPR, ... of one row into registers, zeros from chunk nck
// = K/8 on; the row is 16-byte aligned and K % 8 == 0 (the register-resident
// form is used only then).  FULL: the row is exactly CPL*LPR chunks (K = ldk
// = 8*CPL*LPR), so every lane loads, quantizes and stores all CPL of its
// chunks with no per-chunk test.
template <int CPL, int LPR, bool FULL>
__device__ __forceinline__ void load_row(uint4 (&h)[CPL > 0 ? CPL : 1], const uint16_t* row, int rl,
                                         int nck) {
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int c = rl + u * LPR;
    h[u] = FULL || c < nck ? reinterpret_cast<const uint4*>(row)[c] : uint4{0u, 0u, 0u, 0u};
  }
}

// Mask bytes of the chunks of lane rl (byte u of obs[u / 4] = mask bits of
// chunk rl + u*LPR): the same for every row, so they are gathered once per
// block.
template <int CPL, int LPR, bool FULL>
__device__ __forceinline__ void chunk_mask_bytes(uint32_t (&obs)[(CPL + 3) / 4 > 0 ? (CPL + 3) / 4 : 1],
                                                 const uint32_t* s_bits, int rl, int nch) {
#pragma unroll
  for (int i = 0; i < (CPL + 3) / 4; ++i) obs[i] = 0u;
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int c = rl + u * LPR;
    const uint32_t ob = FULL || c < nch ? (s_bits[c >> 2] >> ((c & 3) * 8)) & 0xffu : 0u;
    obs[u >> 2] |= ob << ((u & 3) * 8);
  }
}

// A lane's entries j = rl, rl + LPR, ... of one row's outlier slice
// (X_O[m][j] = X[m][O_j] for j < |O|, 0 up to opad), held between their
// loads and stores.
struct OutlierRow {
  uint16_t v[4];
};

// One row m (< M) held in registers (CPL > 0): absmax of |x| over the
// regular columns, codes (zero on the outlier columns), stores.  With
// WPR == 4 the block's four waves share the row (block barriers inside).
template <int WPR, int CPL, bool FULL>
__device__ __forceinline__ void quant_row_regs(uint4 (&h)[CPL > 0 ? CPL : 1],
                                               const uint32_t (&obs)[(CPL + 3) / 4 > 0 ? (CPL + 3) / 4 : 1],
                                               const uint16_t* __restrict__ X, int m, int K,
                                               int ldk, int rl, int nch, int total, int opad,
                                               const uint32_t* s_bits, const int* s_pre,
                                               const int* s_olist, bool olist_in_lds, int nw,
                                               uint32_t* s_red, int8_t* __restrict__ Xq,
                                               float* __restrict__ x_scale,
                                               uint16_t* __restrict__ XO) {
  constexpr int LPR = 64 * WPR;
  constexpr int NOB = (CPL + 3) / 4 > 0 ? (CPL + 3) / 4 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* row = X + (size_t)m * K;
  // The mask bytes are the same for every row of the block; left visible,
  // the masks derived from them get hoisted out of the row loop and held in
  // some fifty registers.  An empty asm makes them opaque per row instead.
  uint32_t ob_row[NOB];
#pragma unroll
  for (int i = 0; i < NOB; ++i) {
    ob_row[i] = obs[i];
    asm volatile("" : "+v"(ob_row[i]));
  }
  uint32_t mx2 = 0;  // two packed 16-bit maxima of |x| bits
#pragma unroll
  for (int u = 0; u < CPL; ++u)
    mx2 = pk_max_u16(mx2, chunk_absmax2(h[u], (ob_row[u >> 2] >> ((u & 3) * 8)) & 0xffu));
  uint32_t mx = wave_max(max(mx2 & 0xffffu, mx2 >> 16));
  if (WPR > 1) {
    __syncthreads();  // s_red of the previous row has been read
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    mx = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
  }
  const float a = h2f((uint16_t)mx);
  const float r = a == 0.0f ? 0.0f : 127.0f / a;
  // outlier slice values first (loads from the row just read: cache hits),
  // so that only stores are in flight once the codes start going out
  constexpr int kXoPer = 4;  // slice entries per lane and pass
  OutlierRow xo{{0, 0, 0, 0}};
  const bool xo_one_pass = opad <= kXoPer * LPR;
  if (XO != nullptr && xo_one_pass) {
#pragma unroll
    for (int p = 0; p < kXoPer; ++p) {
      const int j = rl + p * LPR;
      if (j < total) {
        const int k = olist_in_lds ? s_olist[j] : select_outlier(s_bits, s_pre, nw, j);
        xo.v[p] = row[k];
      }
    }
    wait_vmem_all();
  }
  // codes chunk by chunk, each stored at once: the fast quotient, the exact
  // one for a chunk with a value near a half-integer, outlier columns zeroed.
  // Chunk c = rl + u*LPR starts at byte 8c of the row: LPR*8/64 column
  // blocks (of kTileBytes each) after chunk rl.  The stores address the
  // row's 256-row panel (a base the whole wave shares: m is the same in every
  // lane) plus one 32-bit lane offset, kept in a register (left visible, the
  // compiler recomputes the 64-bit tiled offset for every chunk).
  const int mu = __builtin_amdgcn_readfirstlane(m);
  int8_t* xq_panel = Xq + (size_t)(mu >> 8) * kPanelRows * (size_t)ldk;
  uint32_t xoff = (uint32_t)(tiled_offset(mu & 255, (size_t)rl * 8, ldk));
  asm volatile("" : "+v"(xoff));
  constexpr uint32_t kStep = (uint32_t)(LPR * 8 / kTileK * kTileBytes);
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    float dev;
    uint2 q = quant8_fast(h[u], r, &dev);
    if (dev > kTieGuard) q = quant8_exact(h[u], a);
    // the masks again (a few permutes), not held from the absmax pass
    uint32_t obq = (ob_row[u >> 2] >> ((u & 3) * 8)) & 0xffu;
    asm volatile("" : "+v"(obq));
    const ChunkMasks cm = chunk_masks(obq);
    q.x &= ~cm.b[0];
    q.y &= ~cm.b[1];
    if (FULL || rl + u * LPR < nch)
      *reinterpret_cast<uint2*>(xq_panel + (xoff + (uint32_t)u * kStep)) = q;
  }
  if (XO != nullptr) {
    if (xo_one_pass) {
#pragma unroll
      for (int p = 0; p < kXoPer; ++p) {
        const int j = rl + p * LPR;
        if (j < opad) XO[tiled_offset(m, (size_t)j * 2, (size_t)ldk * 2) / 2] = xo.v[p];
      }
    } else {
      // long slices: 8 entries per lane and pass, loads issued together
      constexpr int kXoU = 8;
      for (int j0 = rl; j0 < opad; j0 += kXoU * LPR) {
        uint16_t v[kXoU];
#pragma unroll
        for (int u = 0; u < kXoU; ++u) {
          const int j = j0 + u * LPR;
          v[u] = 0;
          if (j < total) v[u] = row[olist_in_lds ? s_olist[j] : select_outlier(s_bits, s_pre, nw, j)];
        }
#pragma unroll
        for (int u = 0; u < kXoU; ++u) {
          const int j = j0 + u * LPR;
          if (j < opad) XO[tiled_offset(m, (size_t)j * 2, (size_t)ldk * 2) / 2] = v[u];
        }
      }
    }
  }
  if (rl == 0) x_scale[m] = a;
}

// One row m (< M) streamed from memory twice (CPL == 0: long rows, or rows
// that are not 16-byte aligned).
template <int WPR>
__device__ __forceinline__ void quant_row_stream(const uint16_t* __restrict__ X, int m, int K,
                                                 int ldk, int vec, int rl, int nch, int total,
                                                 int opad, const uint32_t* s_bits,
                                                 const int* s_pre, uint32_t* s_red,
                                                 int8_t* __restrict__ Xq,
                                                 float* __restrict__ x_scale,
                                                 uint16_t* __restrict__ XO) {
  constexpr int LPR = 64 * WPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* row = X + (size_t)m * K;
  uint32_t mx2 = 0;
  for (int c = rl; c < nch; c += LPR) {
    const uint4 g = load_chunk(row, c * 8, K, vec != 0);
    const uint32_t ob = (s_bits[c >> 2] >> ((c & 3) * 8)) & 0xffu;
    mx2 = pk_max_u16(mx2, chunk_absmax2(g, ob));
  }
  uint32_t mx = wave_max(max(mx2 & 0xffffu, mx2 >> 16));
  if (WPR > 1) {
    __syncthreads();
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    mx = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
  }
  const float a = h2f((uint16_t)mx);
  const float r = a == 0.0f ? 0.0f : 127.0f / a;
  int8_t* xq_lane = Xq + tiled_offset(m, (size_t)rl * 8, ldk);
  constexpr size_t kStep = (size_t)LPR * 8 / kTileK * kTileBytes;
  int u = 0;
  for (int c = rl; c < nch; c += LPR, ++u) {
    const uint4 g = load_chunk(row, c * 8, K, vec != 0);
    *reinterpret_cast<uint2*>(xq_lane + (size_t)u * kStep) =
        code_chunk(g, m, s_bits[c >> 2], (c & 3) * 8, s_pre[c >> 2], r, a, ldk, XO);
  }
  if (XO != nullptr)
    for (int j = total + rl; j < opad; j += LPR)
      XO[tiled_offset(m, (size_t)j * 2, (size_t)ldk * 2) / 2] = 0;
  if (rl == 0) x_scale[m] = a;
}

// Row pass.  grid = row blocks followed by W_O blocks (16 weight rows each;
// only when WO != nullptr): the row blocks take the machine first, the small
// gathers fill the slots their tail frees.  WPR = waves per row: 1 (a wave
// per row, 4 rows per block and pass, the blocks looping over the rows) or 4
// (the whole block on one row: few rows, or rows too long for one wave's
// registers).  CPL = 8-column chunks per lane held in registers between the
// absmax and the quantize passes (0: re-read the row from L1/L2 instead, for
// rows that are unaligned or too long for any register form).
// Dynamic LDS: 2*nw words plus the O list, olist_cap(ldk) entries: every
// column while the whole stays within 64 KiB (ldk up to ~14.5K, so that even
// |O| = K is gathered through LDS); beyond that, larger |O| falls back to
// select_outlier.
__host__ __device__ inline int olist_cap(int ldk) {
  const int room = 16384 - 2 * (ldk / 32);  // 32-bit words left of 64 KiB
  return ldk < room ? ldk : room;
}

// Row group (of RPB rows) of row block rb: with a multiple of 8*G row blocks
// (G = 64/RPB groups per column-absmax chunk of 64 rows), the groups of chunk
// c go to blocks on XCD c % 8, the XCD that read those rows in the
// column-absmax pass.  (Measured faster in both passes; the L2 is not kept
// across kernels, the row pass fetches all of X again, so the gain is in the
// locality of each XCD's reads, not in L2 hits.)
template <int RPB>
__device__ __forceinline__ int row_group_of(int rb, int n_row_blocks) {
  constexpr int G = kRowChunk / RPB;
  if (n_row_blocks % (8 * G) != 0) return rb;
  const int x = rb & 7, q = rb >> 3;
  return G * (8 * (q / G) + x) + (q % G);
}
constexpr int kWoRows = 16;
constexpr int kRowBlocks = 2048;  // row blocks of the one-wave-per-row form

template <int WPR, int CPL, bool FULL>
__device__ __forceinline__ void quant_rows_body(
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
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // row blocks first, then the W_O blocks (they run in the row blocks' tail)
  const int n_row_blocks = (int)gridDim.x - n_wo_blocks;
  const int rb = (int)blockIdx.x < n_row_blocks ? (int)blockIdx.x : -1;  // -1: a W_O block
  constexpr int RPB = 4 / WPR;               // rows per block and pass
  constexpr int LPR = 64 * WPR;              // lanes per row
  const int rl = (wave % WPR) * 64 + lane;   // lane index within the row
  const int nch = ldk / 8;
  const int mstride = n_row_blocks * RPB;
  int m = (rb >= 0 ? row_group_of<RPB>(rb, n_row_blocks) : rb) * RPB + wave / WPR;
  // the block's first row is loaded before the mask prefix, so the two
  // memory latencies overlap
  uint4 ha[CPL > 0 ? CPL : 1];
  const int nck = K >> 3;  // whole 8-column chunks of a row (K % 8 == 0 when CPL > 0)
  if (CPL > 0 && rb >= 0 && m < M) load_row<CPL, LPR, FULL>(ha, X + (size_t)m * K, rl, nck);
  const int total = load_mask_prefix(mask_bits, nw, s_bits, s_pre);
  const int opad = (total + 63) & ~63;
  // the O list in LDS when it fits (W_O gather, X_O slice)
  int* s_olist = reinterpret_cast<int*>(s_dyn + 2 * nw);
  const bool olist_in_lds = total <= olist_cap(ldk);
  if ((WO != nullptr || XO != nullptr) && olist_in_lds) {
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
    // ---- W_O[n][j] for 16 weight rows: lane jl of row nl makes the 8
    // consecutive entries j0 .. j0+7 (j0 = 8*jl + 128*pass), one 16-byte
    // store; its 8 gathers of int8 codes are issued together.  (More runs per
    // pass measured slower, also at |O| = K.)
    const bool in_lds = olist_in_lds;
    const int n0 = ((int)blockIdx.x - n_row_blocks) * kWoRows;
    const int nl = t >> 4, jl = t & 15;
    const int n = n0 + nl;
    if (n < N) {
      const float aw = w_scale[n];
      for (int j0 = 8 * jl; j0 < opad; j0 += 128) {
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + e;
          q[e] = 0;
          if (j < total) {
            const int k = in_lds ? s_olist[j] : select_outlier(s_bits, s_pre, nw, j);
            q[e] = (int)Wq[tiled_offset(n, (size_t)k, ldk)];
          }
        }
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t lo = j0 + e < total ? dequant_w_half(q[e], aw) : 0u;
          const uint32_t hi = j0 + e + 1 < total ? dequant_w_half(q[e + 1], aw) : 0u;
          h[e / 2] = lo | (hi << 16);
        }
        // 16 bytes at byte 2*j0 of the row: inside one 64-byte block
        *reinterpret_cast<uint4*>(WO + tiled_offset(n, (size_t)j0 * 2, (size_t)ldk * 2) / 2) =
            uint4{h[0], h[1], h[2], h[3]};
      }
    }
    return;
  }

  // ---- rows m, m + mstride, ... (one pass for M <= 4 * kRowBlocks)
  if (CPL > 0) {
    uint32_t obs[(CPL + 3) / 4 > 0 ? (CPL + 3) / 4 : 1];
    chunk_mask_bytes<CPL, LPR, FULL>(obs, s_bits, rl, nch);
    for (bool first = true; m < M; m += mstride, first = false) {
      if (!first) load_row<CPL, LPR, FULL>(ha, X + (size_t)m * K, rl, nck);
      quant_row_regs<WPR, CPL, FULL>(ha, obs, X, m, K, ldk, rl, nch, total, opad, s_bits, s_pre,
                               s_olist, olist_in_lds, nw, s_red, Xq, x_scale, XO);
    }
  } else {
    for (; m < M; m += mstride)
      quant_row_stream<WPR>(X, m, K, ldk, vec, rl, nch, total, opad, s_bits, s_pre, s_red, Xq,
                            x_scale, XO);
  }
}

#define I8MM_QUANT_ROWS_ARGS                                                                   \
  const uint16_t *__restrict__ X, int M, int K, int ldk, int vec, int n_wo_blocks,              \
      const uint32_t *__restrict__ mask_bits, int8_t *__restrict__ Xq,                          \
      float *__restrict__ x_scale, uint16_t *__restrict__ XO, int32_t *__restrict__ n_out,     \
      int32_t *__restrict__ out_idx, const int8_t *__restrict__ Wq,                             \
      const float *__restrict__ w_scale, int N, uint16_t *__restrict__ WO
template <int WPR, int CPL, bool FULL>
__global__ __launch_bounds__(256) void k_quant_rows(I8MM_QUANT_ROWS_ARGS) {
  quant_rows_body<WPR, CPL, FULL>(X, M, K, ldk, vec, n_wo_blocks, mask_bits, Xq, x_scale, XO, n_out,
                            out_idx, Wq, w_scale, N, WO);
}
// The same held to 128 registers (4 waves per SIMD: a wave per row for 16
// rows per CU at once)
template <int WPR, int CPL, bool FULL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_quant_rows4(
    I8MM_QUANT_ROWS_ARGS) {
  quant_rows_body<WPR, CPL, FULL>(X, M, K, ldk, vec, n_wo_blocks, mask_bits, Xq, x_scale, XO, n_out,
                            out_idx, Wq, w_scale, N, WO);
}
#undef I8MM_QUANT_ROWS_ARGS

// ---------------------------------------------------------------- few rows

// The whole activation pass for a few rows (decode shapes, M <= 16) in one
// launch: grid = M workgroups; workgroup m reads all M rows (a few KiB each,
// shared through L2) to form the column absmax and the mask itself, then
// quantizes row m, which it kept in registers.  Workgroup 0 also writes the
// mask words, |O| and the optional mask bytes and O list.  CPT = 8-column
// chunks per thread (ldk <= T * 8 * CPT); MR = rows loaded per chunk (M <=
// MR; rows past M repeat row M-1, so the MR loads are unconditional and in
// flight together, and a single row costs one load, not sixteen: the
// block's loads go through one CU's texture path); rows are 16-byte aligned
// and K % 8 == 0.  Dynamic LDS: 2*nw words.
template <int CPT, int T, int MR>
__global__ __launch_bounds__(T) void k_activation_small(
    const uint16_t* __restrict__ X, int M, int K, int ldk, float threshold,
    uint8_t* __restrict__ mask8, uint32_t* __restrict__ mask_bits, int32_t* __restrict__ n_out,
    int32_t* __restrict__ out_idx, int8_t* __restrict__ Xq, float* __restrict__ x_scale,
    uint16_t* __restrict__ XO) {
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_red[T / 64];
  const int nw = ldk / 32, nch = ldk / 8, nck = K >> 3;
  uint32_t* s_bits = s_dyn;
  int* s_pre = reinterpret_cast<int*>(s_dyn + nw);
  uint8_t* s_ob = reinterpret_cast<uint8_t*>(s_bits);  // mask byte of chunk c (little endian)
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int m = blockIdx.x;
  const uint4* own_row = reinterpret_cast<const uint4*>(X + (size_t)m * K);

  // ---- column absmax over the M rows, mask bytes (strict > threshold)
  uint4 hv[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = t + u * T;
    uint32_t mx[4] = {0u, 0u, 0u, 0u};  // |x| bits, two columns per word
    hv[u] = uint4{0u, 0u, 0u, 0u};
    if (c < nck) {
      // rows past M repeat row M-1 (no effect on the max)
      uint4 rows[MR];
#pragma unroll
      for (int r = 0; r < MR; ++r)
        rows[r] = reinterpret_cast<const uint4*>(X + (size_t)min(r, M - 1) * K)[c];
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        mx[0] = pk_max_u16(mx[0], rows[r].x & 0x7fff7fffu);
        mx[1] = pk_max_u16(mx[1], rows[r].y & 0x7fff7fffu);
        mx[2] = pk_max_u16(mx[2], rows[r].z & 0x7fff7fffu);
        mx[3] = pk_max_u16(mx[3], rows[r].w & 0x7fff7fffu);
      }
      hv[u] = own_row[c];
    }
    if (c < nch) {
      uint32_t ob = 0;  // padding columns (k >= K) are never outliers
      if (c < nck) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t hb = (mx[i >> 1] >> ((i & 1) * 16)) & 0xffffu;
          ob |= (h2f((uint16_t)hb) > threshold ? 1u : 0u) << i;
        }
      }
      s_ob[c] = (uint8_t)ob;
    }
  }
  __syncthreads();
  const int total = mask_prefix_wave0<T>(nw, s_bits, s_pre);
  const int opad = (total + 63) & ~63;

  if (m == 0) {
    for (int w = t; w < nw; w += T) mask_bits[w] = s_bits[w];
    if (mask8 != nullptr)
      for (int k = t; k < K; k += T) mask8[k] = (uint8_t)((s_bits[k >> 5] >> (k & 31)) & 1u);
    if (t == 0 && n_out != nullptr) *n_out = total;
    if (out_idx != nullptr) {
      for (int w = t; w < nw; w += T) {
        uint32_t b = s_bits[w];
        int slot = s_pre[w];
        while (b) {
          out_idx[slot++] = w * 32 + __ffs(b) - 1;
          b &= b - 1;
        }
      }
    }
  }

  // ---- row m: absmax over the regular columns, codes, outlier slice
  uint32_t mx2 = 0;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = t + u * T;
    const uint32_t ob = c < nch ? (uint32_t)s_ob[c] : 0u;
    mx2 = pk_max_u16(mx2, chunk_absmax2(hv[u], ob));
  }
  uint32_t mx = wave_max(max(mx2 & 0xffffu, mx2 >> 16));
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = 0;
#pragma unroll
  for (int w = 0; w < T / 64; ++w) mx = max(mx, s_red[w]);
  const float a = h2f((uint16_t)mx);
  const float r = a == 0.0f ? 0.0f : 127.0f / a;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = t + u * T;
    if (c < nch)
      *reinterpret_cast<uint2*>(Xq + tiled_offset(m, (size_t)c * 8, ldk)) =
          code_chunk(hv[u], m, s_bits[c >> 2], (c & 3) * 8, s_pre[c >> 2], r, a, ldk, XO);
  }
  if (XO != nullptr)
    for (int j = total + t; j < opad; j += T)
      XO[tiled_offset(m, (size_t)j * 2, (size_t)ldk * 2) / 2] = 0;
  if (t == 0) x_scale[m] = a;
}

// counts[i] = number of columns k < K with colmax[k] > thr.t[i]: |O| at each
// threshold, with the comparison k_colmask makes (binary16 maximum widened
// to fp32, strict).  One workgroup per threshold; four independent loads
// per thread and round.
__global__ __launch_bounds__(256) void k_count_above(const uint16_t* __restrict__ colmax, int K,
                                                     CountThresholds thr,
                                                     int32_t* __restrict__ counts) {
  const float t = thr.t[blockIdx.x];
  int c = 0;
  for (int k0 = (int)threadIdx.x; k0 < K; k0 += 4 * 256) {
    uint16_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * 256;
      v[u] = k < K ? colmax[k] : (uint16_t)0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) c += (k0 + u * 256 < K && h2f(v[u]) > t) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  __shared__ int s[4];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) counts[blockIdx.x] = s[0] + s[1] + s[2] + s[3];
}

__global__ void k_zero_half(uint16_t* __restrict__ Y, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    Y[i] = 0;
}

// Y[m][n] = bias[n]: the whole output of an empty contraction with a bias.
__global__ void k_bias_rows(const uint16_t* __restrict__ bias, int64_t M, int64_t N,
                            uint16_t* __restrict__ Y) {
  const int64_t count = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    Y[i] = bias[i % N];
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
                          hipStream_t s, uint16_t* colmax) {
  dim3 grid((ldk + 63) / 64);
  hipLaunchKernelGGL(k_colmask, grid, dim3(256), 0, s, X, part, rc, M, K, ldk, threshold, mask8,
                     mask_bits, colmax);
  return hipGetLastError();
}

template <int WPR, int CPL, bool FULL>
static void launch_qr1(dim3 grid, size_t lds, hipStream_t s, const uint16_t* X, int M, int K,
                       int ldk, int vec, int nwb, const uint32_t* mb, int8_t* Xq, float* xs,
                       uint16_t* XO, int32_t* n_out, int32_t* out_idx, const int8_t* Wq,
                       const float* ws, int N, uint16_t* WO) {
  if constexpr (WPR == 1 && CPL == 10)
    hipLaunchKernelGGL((k_quant_rows4<WPR, CPL, FULL>), grid, dim3(256), lds, s, X, M, K, ldk,
                       vec, nwb, mb, Xq, xs, XO, n_out, out_idx, Wq, ws, N, WO);
  else
    hipLaunchKernelGGL((k_quant_rows<WPR, CPL, FULL>), grid, dim3(256), lds, s, X, M, K, ldk,
                       vec, nwb, mb, Xq, xs, XO, n_out, out_idx, Wq, ws, N, WO);
}
// FULL when the row is exactly the form's CPL*64*WPR chunks (K = ldk)
template <int WPR, int CPL>
static void launch_qr(dim3 grid, size_t lds, hipStream_t s, const uint16_t* X, int M, int K,
                      int ldk, int vec, int nwb, const uint32_t* mb, int8_t* Xq, float* xs,
                      uint16_t* XO, int32_t* n_out, int32_t* out_idx, const int8_t* Wq,
                      const float* ws, int N, uint16_t* WO) {
  if constexpr (CPL > 0) {
    if (K == ldk && ldk == 8 * CPL * 64 * WPR) {
      launch_qr1<WPR, CPL, true>(grid, lds, s, X, M, K, ldk, vec, nwb, mb, Xq, xs, XO, n_out,
                                 out_idx, Wq, ws, N, WO);
      return;
    }
  }
  launch_qr1<WPR, CPL, false>(grid, lds, s, X, M, K, ldk, vec, nwb, mb, Xq, xs, XO, n_out,
                              out_idx, Wq, ws, N, WO);
}

hipError_t launch_quant_rows(const uint16_t* X, int M, int K, int ldk, const uint32_t* mask_bits,
                             int8_t* Xq, float* x_scale, uint16_t* XO, int32_t* n_out,
                             int32_t* out_idx, const int8_t* Wq, const float* w_scale, int N,
                             uint16_t* WO, hipStream_t s) {
  const int vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  // a whole block per row for few rows (keeps the GPU busy) and for rows too
  // long for one wave's registers but not for four waves' (so the row is
  // read once); otherwise a wave per row.  Blocks loop over the rows only
  // beyond kRowBlocks blocks.
  const bool few_rows = M <= 256;
  const bool long_rows = vec && (ldk / 8 + 63) / 64 > 16 && (ldk / 8 + 255) / 256 <= 8;
  const int wpr = (few_rows || long_rows) ? 4 : 1;
  const int n_row_blocks = wpr == 4 ? min(M, kRowBlocks) : min((M + 3) / 4, kRowBlocks);
  const int n_wo_blocks = WO != nullptr ? (N + kWoRows - 1) / kWoRows : 0;
  const size_t lds = (size_t)2 * (ldk / 32) * sizeof(uint32_t) +
                     (WO != nullptr || XO != nullptr ? (size_t)olist_cap(ldk) * sizeof(int) : 0);
  dim3 grid(n_row_blocks + n_wo_blocks);
  const int lanes = 64 * wpr;
  const int cpl_needed = (ldk / 8 + lanes - 1) / lanes;
#define QR(W, C) launch_qr<W, C>(grid, lds, s, X, M, K, ldk, vec, n_wo_blocks, mask_bits, Xq, x_scale, XO, n_out, out_idx, Wq, w_scale, N, WO)
  // rows held in registers need 16-byte loads (aligned X, K % 8 == 0)
  if (!vec) {
    if (wpr == 4) QR(4, 0); else QR(1, 0);
  } else if (wpr == 4) {
    // (register forms sized to the row: every chunk slot held is quantized)
    if (cpl_needed <= 4) QR(4, 4);
    else if (cpl_needed <= 6) QR(4, 6);
    else if (cpl_needed <= 8) QR(4, 8);
    else QR(4, 0);
  } else {
    if (cpl_needed <= 2) QR(1, 2);
    else if (cpl_needed <= 4) QR(1, 4);
    else if (cpl_needed <= 6) QR(1, 6);
    else if (cpl_needed <= 8) QR(1, 8);
    else if (cpl_needed <= 10) QR(1, 10);
    else if (cpl_needed <= 12) QR(1, 12);
    else if (cpl_needed <= 16) QR(1, 16);
    else QR(1, 0);
  }
#undef QR
  return hipGetLastError();
}

bool activation_small_ok(const uint16_t* X, int M, int K, int ldk) {
  return M >= 1 && M <= 16 && (K % 8) == 0 && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
         ldk / 8 <= 1024 * 2;
}

hipError_t launch_activation_small(const uint16_t* X, int M, int K, int ldk, float threshold,
                                   uint8_t* mask8, uint32_t* mask_bits, int32_t* n_out,
                                   int32_t* out_idx, int8_t* Xq, float* x_scale, uint16_t* XO,
                                   hipStream_t s) {
  const int nch = ldk / 8;
  const size_t lds = (size_t)2 * (ldk / 32) * sizeof(uint32_t);
  // one thread per 8-column chunk where it fits: all the loads of a row in
  // one round (1024 threads up to 8192 columns, two chunks each beyond)
#define AS(C, T, R) hipLaunchKernelGGL((k_activation_small<C, T, R>), dim3(M), dim3(T), lds, s, X, M, K, ldk, threshold, mask8, mask_bits, n_out, out_idx, Xq, x_scale, XO)
#define AS_ROWS(C, T) \
  if (M <= 1) AS(C, T, 1); else if (M <= 4) AS(C, T, 4); else AS(C, T, 16)
  if (nch <= 256) {
    AS_ROWS(1, 256);
  } else if (nch <= 1024) {
    AS_ROWS(1, 1024);
  } else {
    AS_ROWS(2, 1024);
  }
#undef AS_ROWS
#undef AS
  return hipGetLastError();
}

hipError_t launch_bias_rows(const uint16_t* bias, int64_t M, int64_t N, uint16_t* Y,
                            hipStream_t s) {
  int64_t blocks = (M * N + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_bias_rows, dim3((unsigned)blocks), dim3(256), 0, s, bias, M, N, Y);
  return hipGetLastError();
}

hipError_t launch_count_above(const uint16_t* colmax, int K, const CountThresholds& thr, int n,
                              int32_t* counts, hipStream_t s) {
  if (n < 1 || n > kMaxCountThresholds || K < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_count_above, dim3(n), dim3(256), 0, s, colmax, K, thr, counts);
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
