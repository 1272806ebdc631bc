// Prefill GEMM of the decomposed int8 matmul on gfx950 matrix cores.
//
//   Y[m,n] = fp16( fp32(C[m,n]) * a_x[m]*a_w[n]/127^2 + sum_j X_O[m,j] W_O[n,j] )
//   C[m,n] = sum_k Xq[m,k] Wq[n,k]                         (int32, exact)
//
// ("LLM.int8() notes", section 2.3: the INT8 term plus the FP16 outlier term;
// "PyTorch 2.9 supports LLM.int8()", section 3: results merged at the end.)
//
// One workgroup = 256x256 output tile, 8 waves, two per SIMD, in a 2x4
// arrangement: each wave owns a 128x64 block held as 4x2
// v_mfma_i32_32x32x32_i8 accumulators (128 AGPRs).  Two waves per SIMD let
// one wave's memory and LDS instructions, which hold up the issuing wave,
// overlap the other wave's MFMAs.  Operands are panel-tiled in memory
// (tile_layout.h), so one 64-byte K step of a 256-row panel is 16 KiB
// contiguous: each wave load instruction reads 1 KiB of whole cache lines.
// Loads go to registers (three rotating one-step buffers, so a load has two
// steps to land) and from there to LDS with swizzled ds_write_b128.  Five LDS
// stages, each written three steps before it is computed: the one computed,
// the next one (its first fragments are read before the current step ends),
// the one written last step, the one being written, and one more, so that a
// workgroup barrier is needed only after every second step; after the loop
// the last two int8 stages are free for the epilogue.
//
// The outlier slice (|O| rounded up to 32 fp16 columns: 64 bytes per row per
// step, the same byte shape as an int8 step) is appended to the same
// pipeline as extra steps on v_mfma_f32_32x32x16_f16.  With at most three
// such steps their operands are prefetched by the int8 loop and the fp16
// products are added in the epilogue; with more, the int32 accumulators are
// rescaled to fp32 and a loop of its own runs the fp16 steps (out of line).
// |O| is read on the device: no host synchronisation.
//
// With few tiles (at most half as many as CUs) each tile is computed by two
// workgroups that split K and exchange int32 partials (see k_gemm_prefill).
//
// MFMA operand convention: lane l supplies row (l%32) of its operand and 16
// bytes of K; both fragments use the same K mapping, so the pairing of K
// indices is consistent whatever order the hardware assigns inside the 16
// bytes (exact for the int8 sum, within fp32 rounding for fp16).  The W
// fragment is the MFMA's first operand, so each lane owns output rows.
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

namespace {

constexpr int BM = kPanelRows;  // 256
constexpr int BN = kPanelRows;
constexpr int NW = 8;           // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int NBUF = 5;  // LDS stages of 256 rows x 64 bytes per operand (160 KiB)
constexpr int WM = 128;  // wave block rows (4 MFMA tiles)
constexpr int WN = 64;   // wave block columns (2 MFMA tiles)
constexpr int TI = WM / 32;
constexpr int TJ = WN / 32;

struct Smem {
  v4i a[NBUF][BM * 4];
  v4i b[NBUF][BN * 4];
};

// LDS slot of 16-byte chunk `ch` (0..3) of tile row `row`.  gfx950 LDS serves
// a 16-byte read in groups of 16 lanes (64 banks, 256 B/clk): 16 consecutive
// rows then hit 16 distinct slots when the chunk is XORed with bits 2..3 of
// the row.
__device__ __forceinline__ int swz(int row, int ch) { return row * 4 + (ch ^ ((row >> 2) & 3)); }

// Source of pipeline step s: int8 steps first, then fp16 outlier steps.
struct Src {
  const char* A;  // panel-tiled; the tile's panel already applied
  const char* B;
  const char* AO;
  const char* BO;
  int nk8;  // number of int8 steps
};

// One step's loads of one wave, in registers: 2 quads per operand.
struct Stage4 {
  v4i v[4];  // n = 2*i + operand
};

// Per-lane constants of the load path.  Load instruction n of wave w reads
// the 1 KiB slice (n/2)*NW + w of the step block of operand n%2 (lane l: 16
// bytes at +16l), i.e. LDS slot q = slice*64 + l, which it writes to the
// swizzled position swz(q / 4, q % 4).
struct LoadMap {
  uint32_t goff[2];  // byte offset in the step block, per slice index i
  int lidx[2];       // v4i index in an LDS stage
};

__device__ __forceinline__ LoadMap load_map(int wave, int lane) {
  LoadMap mp;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = (i * NW + wave) * 64 + lane;
    mp.goff[i] = (uint32_t)q * 16;
    mp.lidx[i] = swz(q >> 2, q & 3);
  }
  return mp;
}

// Block addresses of step s (clamped to the last step by the caller).
__device__ __forceinline__ void step_src(const Src& src, int s, const char*& a, const char*& b) {
  if (s < src.nk8) {
    a = src.A + (size_t)s * kTileBytes;
    b = src.B + (size_t)s * kTileBytes;
  } else {
    a = src.AO + (size_t)(s - src.nk8) * kTileBytes;
    b = src.BO + (size_t)(s - src.nk8) * kTileBytes;
  }
}

// Load instruction n (0..3) of a step into r.
__device__ __forceinline__ void gload1(Stage4& r, const char* a, const char* b, int n,
                                       const LoadMap& mp) {
  const int i = n >> 1;
  r.v[n] = *reinterpret_cast<const v4i*>(((n & 1) ? b : a) + mp.goff[i]);
}

__device__ __forceinline__ void gload_all(Stage4& r, const Src& src, int s, const LoadMap& mp) {
  const char* a;
  const char* b;
  step_src(src, s, a, b);
#pragma unroll
  for (int n = 0; n < 4; ++n) gload1(r, a, b, n, mp);
}

// LDS write n (0..3) of a step's registers into stage buf.
__device__ __forceinline__ void lwrite1(Smem& sm, int buf, const Stage4& r, int n,
                                       const LoadMap& mp) {
  const int i = n >> 1;
  if (n & 1)
    sm.b[buf][mp.lidx[i]] = r.v[n];
  else
    sm.a[buf][mp.lidx[i]] = r.v[n];
}

__device__ __forceinline__ void lwrite_all(Smem& sm, int buf, const Stage4& r, const LoadMap& mp) {
#pragma unroll
  for (int n = 0; n < 4; ++n) lwrite1(sm, buf, r, n, mp);
}

// MFMA operand fragments of one 32-byte K sub-step for the wave's 4x2 tiles.
struct Frag {
  v4i a[TI];
  v4i b[TJ];
};

__device__ __forceinline__ void fload(Frag& f, const Smem& sm, int buf, int kk, int wm0, int wn0,
                                      int lane) {
  const int ch = kk * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < TI; ++i) f.a[i] = sm.a[buf][swz(wm0 + i * 32 + (lane & 31), ch)];
#pragma unroll
  for (int j = 0; j < TJ; ++j) f.b[j] = sm.b[buf][swz(wn0 + j * 32 + (lane & 31), ch)];
}

__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// One MFMA on fragment pair (w, x): the W fragment first.
template <bool F16>
__device__ __forceinline__ void mma1(v16i& acc, const v4i& w, const v4i& x) {
  if constexpr (F16) {
    // acc holds fp32 bit patterns here (reinterpreted in place)
    acc = __builtin_bit_cast(
        v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, w),
                                                     __builtin_bit_cast(v8h, x),
                                                     __builtin_bit_cast(v16f, acc), 0, 0, 0));
  } else {
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(w, x, acc, 0, 0, 0);
  }
}

// One pipeline step kt, in a fixed instruction order (scheduling barriers
// keep the compiler from regrouping it): 8 groups of 2 MFMAs (tiles (i, 0)
// and (i, 1)), groups 0-3 on the sub-step-0 fragments f0 (i = group),
// groups 4-7 on sub-step 1.  Fragment reads: sub-step 1 of this step into f1
// during groups 0-2 (B fragments first), sub-step 0 of the next step into f0
// during groups 4-6 (f0 is free after group 3).  Groups 0-3 also issue one
// load each (step kt+5 into rl) and one LDS write each (step kt+3 from rw,
// loaded during step kt-2).  The barrier comes after every second step
// (sync: odd kt, and the last step of a run): a stage written in step j is
// first read in step j+2, and one of steps j, j+1 ends with a barrier; the
// stage written in step j last held step j-2, read in steps j-3 and j-2, and
// one of steps j-2, j-1 ended with a barrier.  Branch-free otherwise: loads
// past the last step are clamped to it (in bounds, written to stages of
// steps past the last, which are not read again).
template <bool F16>
__device__ __forceinline__ void step(Smem& sm, v16i (&acc)[TI][TJ], Frag& f0, Frag& f1,
                                     Stage4& rl, const Stage4& rw, const Src& src, int kt,
                                     int last, int wm0, int wn0, const LoadMap& mp, int lane,
                                     bool sync) {
  const int cur = kt % NBUF, nxt = (kt + 1) % NBUF, wst = (kt + 3) % NBUF;
  const char* ga;
  const char* gb;
  step_src(src, min(kt + 5, last), ga, gb);
  const int r = lane & 31;
  const int ch1 = 2 + (lane >> 5);  // sub-step 1 chunk
  const int ch0 = (lane >> 5);      // sub-step 0 chunk
  // fragment reads per group (6 per sub-step): b0 b1 | a0 a1 | a2 a3 | -
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const int i = g & 3;
    Frag& fm = g < 4 ? f0 : f1;  // operands of this group's MFMAs
    Frag& fr = g < 4 ? f1 : f0;  // fragments read in this group
    const int rbuf = g < 4 ? cur : nxt;
    const int rch = g < 4 ? ch1 : ch0;
    const int gg = g & 3;
    mma1<F16>(acc[i][0], fm.b[0], fm.a[i]);
    __builtin_amdgcn_sched_barrier(0);
    if (gg == 0) {
      fr.b[0] = sm.b[rbuf][swz(wn0 + r, rch)];
      fr.b[1] = sm.b[rbuf][swz(wn0 + 32 + r, rch)];
    } else if (gg < 3) {
      const int i0 = (gg - 1) * 2;
      fr.a[i0] = sm.a[rbuf][swz(wm0 + i0 * 32 + r, rch)];
      fr.a[i0 + 1] = sm.a[rbuf][swz(wm0 + (i0 + 1) * 32 + r, rch)];
    }
    __builtin_amdgcn_sched_barrier(0);
    mma1<F16>(acc[i][1], fm.b[1], fm.a[i]);
    __builtin_amdgcn_sched_barrier(0);
    if (g < 4) {
      gload1(rl, ga, gb, g, mp);
      lwrite1(sm, wst, rw, g, mp);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // LDS operations complete in order: lgkmcnt(2) leaves only the last two
  // fragment reads (needed from group 2 of the next step on) in flight, so
  // this wave's stage writes have landed before the barrier
  if (sync) {
    __builtin_amdgcn_s_waitcnt(0xc27f);
    __builtin_amdgcn_s_barrier();
  }
}

// Steps kt of [k0, k1) in order; the register buffers rotate with kt mod 3
// (step kt loads step kt+5 into buf[(kt+1)%3] and writes step kt+3 from
// buf[(kt+2)%3]).  Unrolled by three so that the roles are static.
template <bool F16>
__device__ __forceinline__ void run_steps(Smem& sm, v16i (&acc)[TI][TJ], Frag& f0, Frag& f1,
                                          Stage4& b0, Stage4& b1, Stage4& b2, const Src& src,
                                          int k0, int k1, int last, int wm0, int wn0,
                                          const LoadMap& mp, int lane) {
  int kt = k0;
#define SYNC(k) (((k) & 1) != 0 || (k) == k1 - 1)
  // bring kt to a multiple of 3
  while (kt < k1 && kt % 3 != 0) {
    if (kt % 3 == 1)
      step<F16>(sm, acc, f0, f1, b2, b0, src, kt, last, wm0, wn0, mp, lane, SYNC(kt));
    else
      step<F16>(sm, acc, f0, f1, b0, b1, src, kt, last, wm0, wn0, mp, lane, SYNC(kt));
    ++kt;
  }
  for (; kt + 3 <= k1; kt += 3) {
    step<F16>(sm, acc, f0, f1, b1, b2, src, kt, last, wm0, wn0, mp, lane, SYNC(kt));
    step<F16>(sm, acc, f0, f1, b2, b0, src, kt + 1, last, wm0, wn0, mp, lane, SYNC(kt + 1));
    step<F16>(sm, acc, f0, f1, b0, b1, src, kt + 2, last, wm0, wn0, mp, lane, SYNC(kt + 2));
  }
  if (kt < k1) {
    step<F16>(sm, acc, f0, f1, b1, b2, src, kt, last, wm0, wn0, mp, lane, SYNC(kt));
    ++kt;
  }
  if (kt < k1) step<F16>(sm, acc, f0, f1, b2, b0, src, kt, last, wm0, wn0, mp, lane, SYNC(kt));
#undef SYNC
}

// Pipeline prologue: steps 0, 1 and 2 into stages 0, 1 and 2 (through
// buffers 0, 1 and 2), then the loads of steps 3 and 4 into buffers 2 and 0,
// the first fragments of step 0.
__device__ __forceinline__ void prologue(Smem& sm, Frag& f0, Stage4& b0, Stage4& b1, Stage4& b2,
                                         const Src& src, int last, int wm0, int wn0,
                                         const LoadMap& mp, int lane) {
  gload_all(b0, src, 0, mp);
  gload_all(b1, src, min(1, last), mp);
  gload_all(b2, src, min(2, last), mp);
  lwrite_all(sm, 0, b0, mp);
  lwrite_all(sm, 1, b1, mp);
  lwrite_all(sm, 2, b2, mp);
  gload_all(b2, src, min(3, last), mp);
  gload_all(b0, src, min(4, last), mp);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  fload(f0, sm, 0, 0, wm0, wn0, lane);
}

// Accumulator element r of lane `lane` for tile (i, j) holds C at row
// i*32 + lane%32 and column j*32 + acc_col(r, lane) of the wave block: a
// lane owns one row and runs of 4 consecutive columns.
__device__ __forceinline__ int acc_col(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Stores one 32x64 row group of the wave block (fp32, accumulator layout)
// as fp16 Y rows m_base .. m_base+31, columns n_base .. n_base+63, through
// the wave's 4 KiB staging area ys: each lane writes its 4-column runs as
// 8-byte pieces (piece k of row r at position k ^ 2*((r/2)%8), which spreads
// the 32 rows of a write over the banks), then reads whole 16-byte pieces
// back for 128-byte row-segment stores (whole cache lines).
__device__ __forceinline__ void store_rows(const v16f (&y)[TJ], uint16_t* ys,
                                           uint16_t* __restrict__ Y, int M, int N, int m_base,
                                           int n_base, bool vec_store, int lane) {
  const int row = lane & 31;
  const int sw = 2 * ((row >> 1) & 7);
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = j * 8 + q * 2 + (lane >> 5);
      uint2 v;
      v.x = (uint32_t)f2h(y[j][4 * q]) | ((uint32_t)f2h(y[j][4 * q + 1]) << 16);
      v.y = (uint32_t)f2h(y[j][4 * q + 2]) | ((uint32_t)f2h(y[j][4 * q + 3]) << 16);
      *reinterpret_cast<uint2*>(ys + row * WN + (k ^ sw) * 4) = v;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c16 = lane & 7;
  const int n_col = n_base + c16 * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int rl = p * 8 + (lane >> 3);  // row within the 32-row group
    const int m = m_base + rl;
    const int pos = (2 * c16) ^ (2 * ((rl >> 1) & 7));  // even: the pair stays in order
    const v4i v = *reinterpret_cast<const v4i*>(ys + rl * WN + pos * 4);
    if (m < M) {
      if (vec_store && n_col + 8 <= N) {
        // Y is written once and not read again here: stream it past the
        // caches (same HBM write bytes as plain stores, ~2% faster kernel)
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(Y + (size_t)m * N + n_col));
      } else {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n_col + e < N) Y[(size_t)m * N + n_col + e] = h[e];
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tile of workgroup b, in an XCD-aware order: consecutive workgroups go
// round-robin to the 8 XCDs, so each XCD gets a contiguous run of tiles, and
// the tiles are walked in groups of 4 tile-rows so a run shares A and B
// panels in its L2.
__device__ __forceinline__ void tile_of(int b, int M, int N, int& tm, int& tn) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int G = tiles_m * tiles_n;
  const int L = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  constexpr int GROUP = 4;
  const int per_group = GROUP * tiles_n;
  const int first_m = (L / per_group) * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  tm = first_m + (L % per_group) % gsz;
  tn = (L % per_group) / gsz;
}

}  // namespace

// Many outlier columns (more than three fp16 steps).  The int8 steps run
// through the pipeline as in the common path; then the int32 accumulators
// are dequantized into fp32 accumulators and the fp16 steps follow in a
// simpler loop of its own: one step per LDS stage (two stages alternating),
// three register buffers so that each step's loads are issued two steps
// before it is written to LDS, one barrier per step.  Kept out of line so
// that its registers do not shape the common path's allocation.
template <bool BIAS>
__device__ __attribute__((noinline)) void gemm_tile_many_outliers(
    Smem& sm, const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int K,
    int ldk,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale,
    const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
    const int32_t* __restrict__ n_out, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 2) * WM, wn0 = (wave & 3) * WN;
  int tm, tn;
  tile_of(blockIdx.x, M, N, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};

  const int nk8 = ldk / kTileK;
  const int nk16 = (*n_out + 31) / 32;
  Src src;
  src.A = (const char*)Xq + (size_t)tm * nk8 * kTileBytes;
  src.B = (const char*)Wq + (size_t)tn * nk8 * kTileBytes;
  src.AO = (const char*)XO + (size_t)tm * (2 * nk8) * kTileBytes;  // fp16 rows: 2*ldk bytes
  src.BO = (const char*)WO + (size_t)tn * (2 * nk8) * kTileBytes;
  src.nk8 = nk8;

  const LoadMap mp = load_map(__builtin_amdgcn_readfirstlane(wave), lane);
  Stage4 b0, b1, b2;
  if (*n_out < K) {
    // int8 part: the pipeline clamped to the int8 steps (with |O| = K every
    // code is 0 and C = 0: skipped)
    Frag f0, f1;
    const int last8 = nk8 - 1;
    prologue(sm, f0, b0, b1, b2, src, last8, wm0, wn0, mp, lane);
    run_steps<false>(sm, acc, f0, f1, b0, b1, b2, src, 0, nk8, last8, wm0, wn0, mp, lane);
  }

  // fp32 accumulators: fp32(C) * a_x[m] * a_w[n] / 127^2 (+ b[n])
  v16f yf[TI][TJ];
  if constexpr (!BIAS) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const float sx = x_scale[min(m0 + wm0 + i * 32 + (lane & 31), M - 1)];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sw = w_scale[min(n0 + wn0 + j * 32 + acc_col(r, lane), N - 1)] * kInv127Sq;
          yf[i][j][r] = (float)acc[i][j][r] * (sx * sw);
        }
    }
  }

  // fp16 steps st = 0 .. nk16-1 (pipeline steps nk8 + st): step st is in
  // register buffer st % 3 and LDS stage st % 2
  wait_all();
  __syncthreads();  // every wave is done with the int8 stages
  if constexpr (BIAS) {
    // the tile's scales and bias go through stage NBUF-1 (the fp16 steps use
    // stages 0 and 1): per-element global loads of the bias as well would
    // spill registers
    float* s_x = reinterpret_cast<float*>(&sm.a[NBUF - 1][0]);
    float* s_w = s_x + BM;
    float* s_b = s_w + BN;
    if (threadIdx.x < BM) {
      const int t = threadIdx.x;
      s_x[t] = x_scale[min(m0 + t, M - 1)];
      s_w[t] = w_scale[min(n0 + t, N - 1)] * kInv127Sq;
      s_b[t] = h2f(bias[min(n0 + t, N - 1)]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const float sx = s_x[wm0 + i * 32 + (lane & 31)];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn0 + j * 32 + q * 8 + (lane >> 5) * 4;
          const v4f w4 = *reinterpret_cast<const v4f*>(&s_w[c]);
          const v4f b4 = *reinterpret_cast<const v4f*>(&s_b[c]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            yf[i][j][4 * q + e] = (float)acc[i][j][4 * q + e] * (sx * w4[e]) + b4[e];
        }
    }
  }
  gload_all(b0, src, nk8, mp);
  if (nk16 > 1) gload_all(b1, src, nk8 + 1, mp);
  if (nk16 > 2) gload_all(b2, src, nk8 + 2, mp);
  lwrite_all(sm, 0, b0, mp);
  __syncthreads();
  auto f16_step = [&](int st, Stage4& ld, const Stage4& wr) {
    if (st + 3 < nk16) gload_all(ld, src, nk8 + st + 3, mp);
    const int buf = st & 1;
    Frag f[2];  // both sub-steps' fragments read up front
    fload(f[0], sm, buf, 0, wm0, wn0, lane);
    fload(f[1], sm, buf, 1, wm0, wn0, lane);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          yf[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, f[kk].b[j]),
                                                            __builtin_bit_cast(v8h, f[kk].a[i]),
                                                            yf[i][j], 0, 0, 0);
    // stage (st+1) % 2 was last read in step st-1, before the last barrier
    if (st + 1 < nk16) lwrite_all(sm, (st + 1) & 1, wr, mp);
    __syncthreads();
  };
  int st = 0;
  for (; st + 3 <= nk16; st += 3) {
    f16_step(st, b0, b1);
    f16_step(st + 1, b1, b2);
    f16_step(st + 2, b2, b0);
  }
  if (st < nk16) f16_step(st, b0, b1);
  if (st + 1 < nk16) f16_step(st + 1, b1, b2);

  // store fp16 Y through LDS, 4 KiB per wave
  const bool vec_store = (N & 7) == 0;
  uint16_t* ys = reinterpret_cast<uint16_t*>(&sm.a[0][0]) + wave * (32 * WN);
#pragma unroll
  for (int i = 0; i < TI; ++i) store_rows(yf[i], ys, Y, M, N, m0 + wm0 + i * 32, n0 + wn0, vec_store, lane);
}

// nsplit (MODE 0 only): the last nsplit tiles (in workgroup order) are each
// computed by two workgroups, unit u = 0 .. nsplit-1 as workgroups
// nwhole + u (half 0: int8 steps [0, nk8/2)) and nwhole + nsplit + u (half 1:
// [nk8/2, nk8)), after the nwhole = tiles - nsplit whole tiles.  Each half
// stores its int32 partial in cpart; the second to finish (counter ctr[u],
// zeroed by the activation pass of the same call) adds the other's partial,
// an exact integer sum, and runs the epilogue.  Used when the tiles would
// leave most of the GPU idle.
template <int MODE>  // 0: Y (fused epilogue), 1: int32 C
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2))) void
k_gemm_prefill(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int K,
               int ldk,
               const float* __restrict__ x_scale, const float* __restrict__ w_scale,
               const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
               const int32_t* __restrict__ n_out, const uint16_t* __restrict__ bias,
               uint16_t* __restrict__ Y, int32_t* __restrict__ C, int nsplit,
               int32_t* __restrict__ cpart, int32_t* __restrict__ ctr) {
  __shared__ Smem sm;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int nwhole = tiles - nsplit;
  int tb = (int)blockIdx.x, half = 0, su = -1;  // su: split unit of this workgroup
  if ((int)blockIdx.x >= nwhole) {
    const int bb = (int)blockIdx.x - nwhole;
    su = bb % nsplit;
    half = bb / nsplit;
    tb = nwhole + su;
  }
  const bool split = su >= 0;
  if (MODE == 0 && (*n_out + 31) / 32 > 3) {
    // whole tile in one workgroup (half 0 of a split unit is workgroup tb)
    if (half == 0) {
      if (bias != nullptr)
        gemm_tile_many_outliers<true>(sm, Xq, Wq, M, N, K, ldk, x_scale, w_scale, XO, WO, n_out,
                                      bias, Y);
      else
        gemm_tile_many_outliers<false>(sm, Xq, Wq, M, N, K, ldk, x_scale, w_scale, XO, WO, n_out,
                                       nullptr, Y);
    }
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 2) * WM, wn0 = (wave & 3) * WN;
  int tm, tn;
  tile_of(tb, M, N, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};

  const int nk8 = ldk / kTileK;
  const int nk16 = MODE == 0 ? (*n_out + 31) / 32 : 0;
  // this workgroup's int8 steps [k0, k0 + nr); pipeline step s < nr is int8
  // step k0 + s, then come the outlier steps
  const int k0 = half ? nk8 / 2 : 0;
  const int nr = split ? (half ? nk8 - nk8 / 2 : nk8 / 2) : nk8;
  const int last = nr + nk16 - 1;
  Src src;
  src.A = (const char*)Xq + ((size_t)tm * nk8 + k0) * kTileBytes;
  src.B = (const char*)Wq + ((size_t)tn * nk8 + k0) * kTileBytes;
  src.AO = (const char*)XO + (size_t)tm * (2 * nk8) * kTileBytes;  // fp16 rows: 2*ldk bytes
  src.BO = (const char*)WO + (size_t)tn * (2 * nk8) * kTileBytes;
  src.nk8 = nr;

  const LoadMap mp = load_map(__builtin_amdgcn_readfirstlane(wave), lane);
  Stage4 b0, b1, b2;
  Frag f0, f1;
  prologue(sm, f0, b0, b1, b2, src, last, wm0, wn0, mp, lane);

  // ---- int8 x int8 -> int32 over this workgroup's K steps (outlier
  // columns of Xq are zero)
  run_steps<false>(sm, acc, f0, f1, b0, b1, b2, src, 0, nr, last, wm0, wn0, mp, lane);

  if (MODE == 0 && split) {
    // partial of this half, four registers per pass: each lane stores 16
    // bytes, each wave 1 KiB contiguous
    constexpr int kQuads = TI * TJ * 4;
    v4i* mine = reinterpret_cast<v4i*>(cpart) + ((size_t)su * 2 + half) * kQuads * NT + threadIdx.x;
    const v4i* other =
        reinterpret_cast<const v4i*>(cpart) + ((size_t)su * 2 + (half ^ 1)) * kQuads * NT + threadIdx.x;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mine[((i * TJ + j) * 4 + q) * NT] =
              v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    // the flag lives in stage (nr+3) % NBUF, free since the loop's last
    // barrier and overwritten by the epilogue only after its own barrier
    int* s_first = reinterpret_cast<int*>(&sm.a[(nr + 3) % NBUF][0]);
    wait_all();       // this thread's stores have landed
    __syncthreads();  // ... and every other thread's
    if (threadIdx.x == 0) {
      __threadfence();  // the partial is visible device-wide before the count
      const int first = atomicAdd(&ctr[su], 1) == 0;
      if (!first) __threadfence();  // and the other half's is seen after it
      *s_first = first;
    }
    __syncthreads();
    if (*s_first) return;  // the other half finishes the tile
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4i o = other[((i * TJ + j) * 4 + q) * NT];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += o[e];
        }
  }

  if (MODE == 1) {
    wait_all();
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm0 + i * 32 + (lane & 31);
          const int n = n0 + wn0 + j * 32 + acc_col(r, lane);
          if (m < M && n < N) C[(size_t)m * N + n] = acc[i][j][r];
        }
    return;
  }

  // Few outlier steps (at most 3): pipeline steps nr .. nr+2 were written to
  // LDS stages (nr + s) % NBUF by the int8 loop.  Stages (nr + 3) % NBUF and
  // (nr + 4) % NBUF held the last two int8 steps, whose reads ended at the
  // last barrier (the last step of the loop ends with one): the tile's
  // scales go to the second,
  // fp16 Y is staged in the first (4 KiB per wave).  Per 32-row group i:
  // Y = fp32(C)*s read straight from the int32 accumulators, the outlier
  // product accumulated on top, converted to fp16 and stored as 128-byte row
  // segments.
  const bool vec_store = (N & 7) == 0;
  float* s_x = reinterpret_cast<float*>(&sm.a[(nr + NBUF - 1) % NBUF][0]);
  float* s_w = s_x + BM;
  float* s_b = s_w + BN;
  if (threadIdx.x < BM) {
    const int t = threadIdx.x;
    s_x[t] = x_scale[min(m0 + t, M - 1)];
    s_w[t] = w_scale[min(n0 + t, N - 1)] * kInv127Sq;
    s_b[t] = bias != nullptr ? h2f(bias[min(n0 + t, N - 1)]) : 0.0f;
  }
  wait_all();
  __syncthreads();
  const int fs = (nr + 3) % NBUF;
  uint16_t* ys = reinterpret_cast<uint16_t*>(wave < 4 ? &sm.a[fs][0] : &sm.b[fs][0]) +
                 (wave & 3) * (32 * WN);
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    // row group i: scaled int8 part first (its accumulator registers are
    // then free for the fp16 MFMAs), outlier products accumulated on top
    const float sx = s_x[wm0 + i * 32 + (lane & 31)];
    v16f y[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn0 + j * 32 + q * 8 + (lane >> 5) * 4;
        const v4f w4 = *reinterpret_cast<const v4f*>(&s_w[c]);
        const v4f b4 = *reinterpret_cast<const v4f*>(&s_b[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[j][4 * q + e] = (float)acc[i][j][4 * q + e] * (sx * w4[e]) + b4[e];
      }
    for (int st = 0; st < nk16; ++st) {
      const int stg = (nr + st) % NBUF;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        const v8h a = __builtin_bit_cast(v8h, sm.a[stg][swz(wm0 + i * 32 + (lane & 31), ch)]);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const v8h b = __builtin_bit_cast(v8h, sm.b[stg][swz(wn0 + j * 32 + (lane & 31), ch)]);
          y[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, y[j], 0, 0, 0);
        }
      }
    }
    store_rows(y, ys, Y, M, N, m0 + wm0 + i * 32, n0 + wn0, vec_store, lane);
  }
}

hipError_t launch_gemm_prefill(const int8_t* Xq, const int8_t* Wq, int M, int N, int K, int ldk,
                               const float* x_scale, const float* w_scale, const uint16_t* XO,
                               const uint16_t* WO, const int32_t* n_out, const uint16_t* bias,
                               uint16_t* Y, int32_t* C, int nsplit, int32_t* cpart, int32_t* ctr,
                               hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (C != nullptr)
    hipExtLaunchKernelGGL(k_gemm_prefill<1>, dim3(tiles), dim3(NT), 0, s, e0, e1, 0, Xq, Wq, M, N,
                          K, ldk, x_scale, w_scale, XO, WO, n_out, nullptr, Y, C, 0, nullptr,
                          nullptr);
  else
    hipExtLaunchKernelGGL(k_gemm_prefill<0>, dim3(tiles + nsplit), dim3(NT), 0, s, e0, e1, 0,
                          Xq, Wq, M, N, K, ldk, x_scale, w_scale, XO, WO, n_out, bias, Y, C,
                          nsplit, cpart, ctr);
  return hipGetLastError();
}

int gemm_prefill_nsplit(int M, int N, int ldk, int n_cu) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (ldk / kTileK < 32 || n_cu <= 0) return 0;  // short K: the exchange would not pay
  // Every tile split when the tiles fill at most half of the CUs (one
  // workgroup per CU).  Splitting only the tiles of a partly filled last
  // round measured no faster: the exchange of the int32 partials (HBM-bound
  // when all the split units end together) costs about what it saves.
  return 2 * tiles <= n_cu ? tiles : 0;
}

}  // namespace i8mm
