// Prefill GEMM of the decomposed int8 matmul on gfx950 matrix cores.
//
//   Y[m,n] = fp16( fp32(C[m,n]) * a_x[m]*a_w[n]/127^2 + b[n] + sum_j X_O[m,j] W_O[n,j] )
//   C[m,n] = sum_k Xq[m,k] Wq[n,k]                         (int32, exact)
//
// ("LLM.int8() notes", section 2.3: the INT8 term plus the FP16 outlier term;
// "PyTorch 2.9 supports LLM.int8()", section 3: results merged at the end.)
//
// One workgroup = 256x256 output tile, 4 waves, one per SIMD, each owning a
// 128x128 block held as 4x4 v_mfma_i32_32x32x32_i8 accumulators (all 256
// AGPRs).  Per 32-byte K sub-step a wave reads 4 + 4 fragments from LDS for
// 16 MFMAs.  Operands are panel-tiled in memory (tile_layout.h): one 64-byte K
// step of a 256-row panel is 16 KiB contiguous.
//
// Loads go straight from L2 into LDS (buffer_load_dwordx4 ... lds): each load
// instruction fills 1 KiB of a stage, its lanes reading the 16-byte chunks
// that the XOR swizzle of the fragment reads puts there.  Four stages of
// 32 KiB (A block, then B block) form a ring; step kt+4's loads are issued
// while step kt computes, and one workgroup barrier per step both publishes
// the next stage and frees the one just consumed (see step()).  The loads are
// branch-free: every buffer resource ends where its operand's valid steps
// end, so the loads of steps past the last one fall outside it and fetch
// nothing, and every step waits for the same load count.  (Conditional loads
// measured ~20% slower: the scalar branches around them stall the issuing
// wave while its MFMAs drain.)
//
// The outlier slice (|O| rounded up to 32 fp16 columns: 64 bytes per row per
// step, the same byte shape as an int8 step) follows the int8 steps in the
// same pipeline.  With at most three such steps they are only loaded by the
// int8 loop, and the epilogue multiplies them from LDS per 32-row group
// (v_mfma_f32_32x32x16_f16) onto fp32(C)*s + b; with more, the tile takes a
// path of its own that rescales the int32 accumulators to fp32 in place and
// continues the pipeline over the fp16 steps.  |O| is read on the device: no
// host synchronisation.
//
// Tiles of a round that would fill at most half of the CUs (a short last
// round, or all of them when there are few) are computed as two 256x128
// halves each (wave blocks of 128x64), which all run at once in half the time
// of a whole tile (see k_gemm_prefill).
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
constexpr int NW = 4;           // waves per workgroup, one per SIMD
constexpr int NT = 64 * NW;
constexpr int NS = 4;                          // LDS stages
constexpr int kStage = 2 * kTileBytes;         // A block then B block: 32 KiB
constexpr int kScaleOff = NS * kStage;         // s_x[256], s_w[256], s_b[256], flag
constexpr int kLds = kScaleOff + 3 * 1024 + 16;
constexpr int WM = 128;                        // wave block rows
constexpr int TI = WM / 32;
constexpr int kRsrcWord3 = 0x00020000;         // raw byte buffer
constexpr int kLoadsA = kTileBytes / 1024 / NW;  // per wave and step: 4
// TJ (template parameter below): 32-column fragments of a wave block, 4 for a
// whole 256x256 tile (wave block 128x128), 2 for a half tile of 256x128
// (wave block 128x64, whose B block is the matching half of the B step block)

// s_waitcnt immediate: vmcnt <= vm, lgkmcnt <= lgkm, expcnt not waited on
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

template <int TJ>
struct Frag {
  v4i a[TI];
  v4i b[TJ];
};

// Per-tile pipeline state, all wave-uniform except the per-lane offsets.
struct Pipe {
  __amdgpu_buffer_rsrc_t A;   // int8 step blocks (step s at s*16 KiB)
  __amdgpu_buffer_rsrc_t B;
  __amdgpu_buffer_rsrc_t AO;  // fp16 outlier step blocks
  __amdgpu_buffer_rsrc_t BO;
  int nk8;                    // int8 steps; steps nk8 .. last are outlier steps
  int last;                   // last pipeline step
  uint32_t goff;              // lane's byte offset in a step block for load 0
  uint32_t boff;              // start of the B rows in a step block (half tile 1: 8 KiB)
  uint32_t ldsw;              // wave's byte offset in an operand's stage block
  uint32_t ra[2];             // fragment read offsets in a stage, sub-step kk, A
  uint32_t rb[2];             // ... B (includes the 16 KiB of the A block)
};

template <int TJ>
__device__ __forceinline__ void make_pipe(Pipe& p, const int8_t* Xq, const int8_t* Wq,
                                          const uint16_t* XO, const uint16_t* WO, int tm, int tn,
                                          int h, int nk8, int k0, int n8, int n16, int wave,
                                          int lane) {
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * (32 * TJ);
  // each resource spans exactly the steps this workgroup consumes
  p.A = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)Xq + ((size_t)tm * nk8 + k0) * kTileBytes), 0, n8 * kTileBytes,
      kRsrcWord3);
  p.B = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)Wq + ((size_t)tn * nk8 + k0) * kTileBytes), 0, n8 * kTileBytes,
      kRsrcWord3);
  // fp16 rows are 2*ldk bytes: panel t starts at t * 2*nk8 blocks
  p.AO = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)XO + (size_t)tm * (2 * nk8) * kTileBytes), 0, n16 * kTileBytes,
      kRsrcWord3);
  p.BO = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)WO + (size_t)tn * (2 * nk8) * kTileBytes), 0, n16 * kTileBytes,
      kRsrcWord3);
  p.nk8 = n8;
  p.last = n8 + n16 - 1;
  // load q of wave w fills LDS slots [(4q+w)*64, +64) of the operand block;
  // lane l fills slot s = base + l: row s/4, stored chunk s%4, which holds
  // logical chunk (s%4) ^ ((row/4)%4) (the swizzle of the fragment reads)
  const int c = (lane & 3) ^ ((lane >> 4) & 3);
  p.goff = (uint32_t)(wave * 1024 + (lane >> 2) * 64 + c * 16);
  // B rows h*128 .. of the panel: the same swizzle (128 rows = 32 whole
  // groups of four)
  p.boff = (uint32_t)(h * (kTileBytes / 2));
  p.ldsw = (uint32_t)(wave * 1024);
  // fragment read of tile row r, chunk ch: slot r*4 + (ch ^ ((r/4)%4)); 16
  // consecutive rows hit 16 distinct slots of the 64 banks
  const int r = lane & 31, sw = (r >> 2) & 3;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int ch = (kk * 2 + (lane >> 5)) ^ sw;
    p.ra[kk] = (uint32_t)((wm0 + r) * 64 + ch * 16);
    p.rb[kk] = (uint32_t)(kTileBytes + (wn0 + r) * 64 + ch * 16);
  }
}

// Buffer resource and byte offset of operand b of pipeline step s (past the
// last step: outside the outlier resource, so the load fetches nothing).
struct Blk {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off;
};
__device__ __forceinline__ Blk blk(const Pipe& p, int s, bool b) {
  const uint32_t o = b ? p.boff : 0u;
  if (s < p.nk8) return Blk{b ? p.B : p.A, (uint32_t)s * kTileBytes + o};
  return Blk{b ? p.BO : p.AO, (uint32_t)(s - p.nk8) * kTileBytes + o};
}

// Load q (0..3; 0..1 for the B half of a half tile) of operand b of step s
// into stage s%NS.
__device__ __forceinline__ void gload(char* lds, const Pipe& p, const Blk& src, int s, bool b,
                                      int q) {
  char* dst = lds + (s & (NS - 1)) * kStage + (b ? kTileBytes : 0) + q * 4096 + p.ldsw;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (__attribute__((address_space(3))) void*)dst,
                                           16, p.goff, src.off + q * 4096, 0, 0);
}

__device__ __forceinline__ v4i lread(const char* lds, uint32_t off) {
  return *reinterpret_cast<const v4i*>(lds + off);
}

template <bool F16>
__device__ __forceinline__ void mma1(v16i& acc, const v4i& w, const v4i& x) {
  if constexpr (F16) {
    // acc holds fp32 bit patterns here (rescaled in place)
    acc = __builtin_bit_cast(
        v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, w),
                                                     __builtin_bit_cast(v8h, x),
                                                     __builtin_bit_cast(v16f, acc), 0, 0, 0));
  } else {
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(w, x, acc, 0, 0, 0);
  }
}

// Fragment read n (0 .. TI+TJ-1) of sub-step kk in the order the MFMAs need
// them: b0 a0 b1 .. b[TJ-1] a1 .. a3 (MFMA t uses a[t/TJ], b[t%TJ]).
template <int TJ>
__device__ __forceinline__ void fread1(Frag<TJ>& f, const char* lds, uint32_t sbase, const Pipe& p,
                                       int kk, int n) {
  if (n == 0)
    f.b[0] = lread(lds, sbase + p.rb[kk]);
  else if (n == 1)
    f.a[0] = lread(lds, sbase + p.ra[kk]);
  else if (n <= TJ)
    f.b[n - 1] = lread(lds, sbase + p.rb[kk] + (n - 1) * 2048);
  else
    f.a[n - TJ] = lread(lds, sbase + p.ra[kk] + (n - TJ) * 2048);
}

// Per step and wave: kLoadsA loads of the A block, TJ of the B block (the
// whole 16 KiB block for TJ = 4, its half for TJ = 2).
template <int TJ>
constexpr int loads_per_step() {
  return kLoadsA + TJ;
}

// The MFMA after which load q of n is issued: the loads are spread over the
// MFMAs that follow the fragment reads.
template <int TJ>
constexpr int load_slot(int q, int n) {
  return (TI + TJ) + ((q + 1) * (TI * TJ - (TI + TJ)) - 1) / n;
}

// One pipeline step kt, in a fixed instruction order (scheduling barriers
// keep the compiler from regrouping it):
//   phase 1: TI*TJ MFMAs on f0 (sub-step 0 of kt); after each of the first
//            TI+TJ a fragment read of f1 (sub-step 1 of kt, stage kt%4); after
//            the rest, the B loads of step kt+3 into stage (kt+3)%4.
//   wait + barrier: this wave's loads of step kt+1 have landed (the loads of
//            steps kt+2, kt+3 may still be in flight) and its fragment reads
//            are done; after the barrier every wave's are, so stage (kt+1)%4
//            is complete and stage kt%4 is free.
//   phase 2: TI*TJ MFMAs on f1; reads of f0 (sub-step 0 of kt+1, stage
//            (kt+1)%4); A loads of step kt+4 into stage kt%4.
// Loads complete in issue order, so the loads of step j are the A half (phase
// 2 of step j-4) then the B half (phase 1 of step j-3), and at the barrier of
// step kt exactly the loads of steps kt+2, kt+3 were issued after step kt+1's.
template <bool F16, int TJ>
__device__ __forceinline__ void step(char* lds, v16i (&acc)[TI][TJ], Frag<TJ>& f0, Frag<TJ>& f1,
                                     const Pipe& p, int kt) {
  constexpr int MT = TI * TJ, NR = TI + TJ;
  const uint32_t cur = (uint32_t)(kt & (NS - 1)) * kStage;
  const uint32_t nxt = (uint32_t)((kt + 1) & (NS - 1)) * kStage;
  const int sb = kt + NS - 1, sa = kt + NS;
  const Blk gsb = blk(p, sb, true);
  const Blk gsa = blk(p, sa, false);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    mma1<F16>(acc[t / TJ][t % TJ], f0.b[t % TJ], f0.a[t / TJ]);
    __builtin_amdgcn_sched_barrier(0);
    if (t < NR) {
      fread1<TJ>(f1, lds, cur, p, 1, t);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < TJ; ++q)
      if (t == load_slot<TJ>(q, TJ)) {
        gload(lds, p, gsb, sb, true, q);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * loads_per_step<TJ>(), 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    mma1<F16>(acc[t / TJ][t % TJ], f1.b[t % TJ], f1.a[t / TJ]);
    __builtin_amdgcn_sched_barrier(0);
    if (t < NR) {
      fread1<TJ>(f0, lds, nxt, p, 0, t);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q)
      if (t == load_slot<TJ>(q, kLoadsA)) {
        gload(lds, p, gsa, sa, false, q);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
}

template <bool F16, int TJ>
__device__ __forceinline__ void run_steps(char* lds, v16i (&acc)[TI][TJ], Frag<TJ>& f0,
                                          Frag<TJ>& f1, const Pipe& p, int k0, int k1) {
  int kt = k0;
  for (; kt + 2 <= k1; kt += 2) {
    step<F16, TJ>(lds, acc, f0, f1, p, kt);
    step<F16, TJ>(lds, acc, f0, f1, p, kt + 1);
  }
  if (kt < k1) step<F16, TJ>(lds, acc, f0, f1, p, kt);
}

// Pipeline prologue: loads of steps 0 .. NS-2 and the A half of step NS-1
// (the steady state's lead), then step 0 landed everywhere and f0 holds its
// sub-step 0.
template <int TJ>
__device__ __forceinline__ void prologue(char* lds, Frag<TJ>& f0, const Pipe& p) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const Blk a = blk(p, s, false);
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q) gload(lds, p, a, s, false, q);
    if (s < NS - 1) {
      const Blk b = blk(p, s, true);
#pragma unroll
      for (int q = 0; q < TJ; ++q) gload(lds, p, b, s, true, q);
    }
  }
  // issued after step 0's loads: steps 1 .. NS-2 and A of NS-1
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * loads_per_step<TJ>() + kLoadsA, 0));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int n = 0; n < TI + TJ; ++n) fread1<TJ>(f0, lds, 0, p, 0, n);
}

// Accumulator element r of lane `lane` for tile (i, j) holds C at row
// i*32 + lane%32 and column j*32 + acc_col(r, lane) of the wave block: a
// lane owns one row and runs of 4 consecutive columns.
__device__ __forceinline__ int acc_col(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
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

// Stores rows m_base .. +31, columns n_base .. +32*TJ-1 of Y from y (fp32,
// accumulator layout) through the wave's 8 KiB staging area ys (256-byte
// rows): each lane writes its 4-column runs as 8-byte pieces (piece e of row
// r at position e ^ 2*((r/2)%16), which spreads the rows of a write over the
// banks), then reads back whole 16-byte pieces for row-segment stores of
// 64*TJ bytes.  INTERIOR: the whole block lies inside Y and N % 8 == 0, so the
// stores need no checks (branches around every store measured a large part
// of the epilogue).
template <int TJ, bool INTERIOR>
__device__ __forceinline__ void store_rows(const v16f (&y)[TJ], char* ys, uint16_t* __restrict__ Y,
                                           int M, int N, int m_base, int n_base, bool vec,
                                           int lane) {
  const int row = lane & 31;
  const int sw = 2 * ((row >> 1) & 15);
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = j * 8 + q * 2 + (lane >> 5);
      uint2 v;
      v.x = f2h2(y[j][4 * q], y[j][4 * q + 1]);
      v.y = f2h2(y[j][4 * q + 2], y[j][4 * q + 3]);
      *reinterpret_cast<uint2*>(ys + row * 256 + (e ^ sw) * 8) = v;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int PR = 4 * TJ;   // 16-byte pieces of a row segment
  constexpr int RPP = 64 / PR;  // rows per pass
  const int c = lane % PR;
  if constexpr (INTERIOR) {
    // a uniform block base and one per-lane element offset for every pass
    uint16_t* yb = Y + (size_t)m_base * N + n_base;
    const uint32_t loff = (uint32_t)((lane / PR) * N + c * 8);
#pragma unroll
    for (int pp = 0; pp < 32 / RPP; ++pp) {
      const int rl = pp * RPP + lane / PR;
      const int pos = (2 * c) ^ (2 * ((rl >> 1) & 15));  // even: the pair stays in order
      const v4i v = *reinterpret_cast<const v4i*>(ys + rl * 256 + pos * 8);
      // Y is written once and not read again here: stream it past the caches
      __builtin_nontemporal_store(
          v, reinterpret_cast<v4i*>(yb + (size_t)(pp * RPP) * N + loff));
    }
  } else {
    const int n_col = n_base + c * 8;
#pragma unroll
    for (int pp = 0; pp < 32 / RPP; ++pp) {
      const int rl = pp * RPP + lane / PR;
      const int m = m_base + rl;
      const int pos = (2 * c) ^ (2 * ((rl >> 1) & 15));
      const v4i v = *reinterpret_cast<const v4i*>(ys + rl * 256 + pos * 8);
      if (m < M) {
        if (vec && n_col + 8 <= N) {
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(Y + (size_t)m * N + n_col));
        } else {
          const uint16_t* hh = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n_col + e < N) Y[(size_t)m * N + n_col + e] = hh[e];
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Many outlier columns (more than NS-1 fp16 steps): the whole tile in one
// workgroup; the int8 steps, then the accumulators rescaled in place to fp32
// (fp32(C)*s + b, the order of the few-outlier epilogue) and the fp16 steps
// continued through the same pipeline.  With |O| = K every code is 0 and C =
// 0: the int8 steps are skipped.  A branch of its own at the kernel's start,
// so nothing of the common path is live in it.
__device__ __forceinline__ void gemm_tile_many(char* lds, const int8_t* __restrict__ Xq,
                                               const int8_t* __restrict__ Wq, int M, int N, int K,
                                               int ldk, const uint16_t* __restrict__ XO,
                                               const uint16_t* __restrict__ WO, int n_out,
                                               uint16_t* __restrict__ Y, int tm, int tn) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int TJ = 4;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * (32 * TJ);
  const int m0 = tm * BM, n0 = tn * BN;
  const float* s_x = reinterpret_cast<const float*>(lds + kScaleOff);
  const float* s_w = s_x + BM;
  const float* s_b = s_w + BN;
  const int nk8 = ldk / kTileK;
  const int nk16 = (n_out + 31) / 32;
  const int n8 = n_out < K ? nk8 : 0;
  Pipe p;
  make_pipe<TJ>(p, Xq, Wq, XO, WO, tm, tn, 0, nk8, 0, n8, nk16, wave, lane);
  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};
  Frag<TJ> f0, f1;
  prologue(lds, f0, p);
  run_steps<false, TJ>(lds, acc, f0, f1, p, 0, n8);
  // step n8's sub-step-0 fragments are read again after the rescale (its
  // stage is complete and nothing overwrites it before step n8 runs), so
  // the fragment registers are free during it
  f0 = Frag<TJ>{};
  // one column quad at a time (its scales and biases read once, applied to
  // the four row groups), so that few registers are live beside the
  // accumulators
  float sx[TI];
#pragma unroll
  for (int i = 0; i < TI; ++i) sx[i] = s_x[wm0 + i * 32 + (lane & 31)];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = wn0 + j * 32 + q * 8 + (lane >> 5) * 4;
      const v4f w4 = *reinterpret_cast<const v4f*>(&s_w[c]);
      const v4f b4 = *reinterpret_cast<const v4f*>(&s_b[c]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j][4 * q + e] =
              __float_as_int((float)acc[i][j][4 * q + e] * (sx[i] * w4[e]) + b4[e]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
  for (int n = 0; n < TI + TJ; ++n)
    fread1<TJ>(f0, lds, (uint32_t)(n8 & (NS - 1)) * kStage, p, 0, n);
  run_steps<true, TJ>(lds, acc, f0, f1, p, n8, n8 + nk16);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const bool vec = (N & 7) == 0;
  char* ys = lds + wave * 8192;
  const bool interior = vec && m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    v16f y[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) y[j] = __builtin_bit_cast(v16f, acc[i][j]);
    if (interior)
      store_rows<TJ, true>(y, ys, Y, M, N, m0 + wm0 + i * 32, n0 + wn0, vec, lane);
    else
      store_rows<TJ, false>(y, ys, Y, M, N, m0 + wm0 + i * 32, n0 + wn0, vec, lane);
  }
}

// Few outlier steps (at most NS-1): pipeline steps nr .. nr+nk16-1 sit in
// LDS stages (nr+st)%NS, loaded by the int8 loop; stage (nr-1)%NS, the last
// int8 step's, is free once every load has landed (the loads past the last
// step that targeted it fetched nothing) and stages Y (8 KiB per wave).  Per
// 32-row group i: Y = fp32(C)*s + b straight from the int32 accumulators,
// the outlier products accumulated on top, fp16 rows stored.
template <int TJ, bool INTERIOR, bool OUTLIERS>
__device__ __forceinline__ void epilogue_few(char* lds, v16i (&acc)[TI][TJ], const Pipe& p, int nr,
                                             int nk16, char* ys, uint16_t* __restrict__ Y, int M,
                                             int N, int m0, int n0, bool vec) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * (32 * TJ);
  const float* s_x = reinterpret_cast<const float*>(lds + kScaleOff);
  const float* s_w = s_x + BM;
  const float* s_b = s_w + BN;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const float sx = s_x[wm0 + i * 32 + (lane & 31)];
    // the column scales and biases are read again for every row group: held
    // across the groups they would take 32*TJ registers and force spills
    int cb = wn0 + (lane >> 5) * 4;
    asm volatile("" : "+v"(cb));
    // fp32(C)*s + b written back into the group's own accumulator registers
    // (as fp32 bit patterns): the outlier MFMAs then accumulate where the
    // values already are (a separate fp32 copy measured ~4x slower, the
    // compiler moving it between register files around every MFMA)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = cb + j * 32 + q * 8;
        const v4f w4 = *reinterpret_cast<const v4f*>(&s_w[c]);
        const v4f b4 = *reinterpret_cast<const v4f*>(&s_b[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j][4 * q + e] =
              __float_as_int((float)acc[i][j][4 * q + e] * (sx * w4[e]) + b4[e]);
      }
    // at least one step when OUTLIERS (tiles without outlier steps take the
    // form without the loop: a loop that may run no times makes the compiler
    // copy the rescaled group into the MFMA registers twice)
    if constexpr (OUTLIERS) {
    int st = 0;
    do {
      const uint32_t sb = (uint32_t)((nr + st) & (NS - 1)) * kStage;
      // all of the step's fragments first, so the reads overlap instead of
      // each MFMA waiting on the one read before it
      v4i a[2], bb[2][TJ];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        a[kk] = lread(lds, sb + p.ra[kk] + i * 2048);
#pragma unroll
        for (int j = 0; j < TJ; ++j) bb[kk][j] = lread(lds, sb + p.rb[kk] + j * 2048);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_bit_cast(
              v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(v8h, bb[kk][j]), __builtin_bit_cast(v8h, a[kk]),
                        __builtin_bit_cast(v16f, acc[i][j]), 0, 0, 0));
    } while (++st < nk16);
    }
    v16f y[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) y[j] = __builtin_bit_cast(v16f, acc[i][j]);
    store_rows<TJ, INTERIOR>(y, ys, Y, M, N, m0 + wm0 + i * 32, n0 + wn0, vec, lane);
  }
}

// The tile's work after the scales are staged: the int8 pipeline, then the
// C store (MODE 1) or the fused epilogue.  TJ = 4: the whole tile (n0 = its
// first column); TJ = 2: the half tile h, columns n0 = tile start + 128h on.
template <int MODE, int TJ>
__device__ __forceinline__ void tile_work(char* lds, const int8_t* __restrict__ Xq,
                                          const int8_t* __restrict__ Wq, int M, int N, int nk8,
                                          int nk16, const uint16_t* __restrict__ XO,
                                          const uint16_t* __restrict__ WO,
                                          uint16_t* __restrict__ Y, int32_t* __restrict__ C,
                                          int tm, int tn, int h, int m0, int n0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * (32 * TJ);

  // pipeline step s < nk8 is int8 step s, then come the outlier steps
  const int nr = nk8;
  Pipe p;
  make_pipe<TJ>(p, Xq, Wq, XO, WO, tm, tn, h, nk8, 0, nr, nk16, wave, lane);

  v16i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16i{};

  Frag<TJ> f0, f1;
  prologue<TJ>(lds, f0, p);
  // int8 x int8 -> int32 over K (outlier columns of Xq are zero); the loads
  // of the outlier steps ride along
  run_steps<false, TJ>(lds, acc, f0, f1, p, 0, nr);

  if constexpr (MODE == 1) {
    __builtin_amdgcn_s_waitcnt(0);
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

  // few outlier steps: the epilogue (see epilogue_few)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const bool vec = (N & 7) == 0;
  char* ys = lds + ((nr + NS - 1) & (NS - 1)) * kStage + wave * 8192;
  // a uniform branch: tiles wholly inside Y (all but the ragged edge) store
  // without checks
  if (vec && m0 + BM <= M && n0 + 64 * TJ <= N) {
    if (nk16 > 0)
      epilogue_few<TJ, true, true>(lds, acc, p, nr, nk16, ys, Y, M, N, m0, n0, vec);
    else
      epilogue_few<TJ, true, false>(lds, acc, p, nr, nk16, ys, Y, M, N, m0, n0, vec);
  } else {
    if (nk16 > 0)
      epilogue_few<TJ, false, true>(lds, acc, p, nr, nk16, ys, Y, M, N, m0, n0, vec);
    else
      epilogue_few<TJ, false, false>(lds, acc, p, nr, nk16, ys, Y, M, N, m0, n0, vec);
  }
}

}  // namespace

// Workgroups 0 .. nwhole-1 compute whole tiles (in workgroup order), then
// come nhalf half-tile pairs (MODE 0 only): each of the last nhalf tiles is
// computed as two 256x128 halves by two workgroups 8 apart (so on the same
// XCD, sharing the A panel in its L2).  Used for a last round of whole tiles
// that would fill at most half of the CUs (its halves then all run at once,
// in half the time), and for every tile when there are at most half as many
// tiles as CUs.  (Halves measured faster there than splitting K between two
// workgroups that exchange int32 partials: no exchange, and the A panel is
// read from the L2 twice instead.)
template <int MODE>  // 0: Y (fused epilogue), 1: int32 C
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void
k_gemm_prefill(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int K,
               int ldk, const float* __restrict__ x_scale, const float* __restrict__ w_scale,
               const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
               const int32_t* __restrict__ n_out, const uint16_t* __restrict__ bias,
               uint16_t* __restrict__ Y, int32_t* __restrict__ C, int nhalf) {
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  // ht: a half tile, `half` its column half
  int tb = (int)blockIdx.x, half = 0;
  bool ht = false;
  const int nwhole = tiles - nhalf;
  if (tb >= nwhole) {
    // groups of 8 tiles: workgroups bb and bb + 8 of a group of 16 take the
    // two halves of one tile; the last nhalf % 8 tiles in adjacent pairs
    const int bb = tb - nwhole;
    const int g16 = 16 * (nhalf / 8);
    int t;
    if (bb < g16) {
      t = (bb / 16) * 8 + bb % 8;
      half = (bb / 8) & 1;
    } else {
      t = 8 * (nhalf / 8) + (bb - g16) / 2;
      half = (bb - g16) & 1;
    }
    tb = nwhole + t;
    ht = true;
  }
  int tm, tn;
  tile_of(tb, M, N, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN + (ht ? half * (BN / 2) : 0);

  // the unit's scales (w_scale already divided by 127^2) and biases, read by
  // the epilogue after the loop's barriers have published them
  float* s_x = reinterpret_cast<float*>(lds + kScaleOff);
  float* s_w = s_x + BM;
  float* s_b = s_w + BN;
  if (MODE == 0) {
    const int t = threadIdx.x;
    s_x[t] = x_scale[min(m0 + t, M - 1)];
    s_w[t] = w_scale[min(n0 + t, N - 1)] * kInv127Sq;
    s_b[t] = bias != nullptr ? h2f(bias[min(n0 + t, N - 1)]) : 0.0f;
  }

  const int nk8 = ldk / kTileK;
  const int nk16 = MODE == 0 ? (*n_out + 31) / 32 : 0;
  if (MODE == 0 && nk16 > NS - 1) {
    // whole tile in one workgroup: half 0 of a half-tile pair (its scales
    // start at the tile's first column) computes it
    __syncthreads();  // the tile's scales are in LDS
    if (half == 0) gemm_tile_many(lds, Xq, Wq, M, N, K, ldk, XO, WO, *n_out, Y, tm, tn);
    return;
  }
  if constexpr (MODE == 0) {
    if (ht) {
      tile_work<MODE, 2>(lds, Xq, Wq, M, N, nk8, nk16, XO, WO, Y, C, tm, tn, half, m0, n0);
      return;
    }
  }
  tile_work<MODE, 4>(lds, Xq, Wq, M, N, nk8, nk16, XO, WO, Y, C, tm, tn, 0, m0, n0);
}

hipError_t launch_gemm_prefill(const int8_t* Xq, const int8_t* Wq, int M, int N, int K, int ldk,
                               const float* x_scale, const float* w_scale, const uint16_t* XO,
                               const uint16_t* WO, const int32_t* n_out, const uint16_t* bias,
                               uint16_t* Y, int32_t* C, int nhalf, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (nhalf < 0 || nhalf > tiles) return hipErrorInvalidValue;
  if (C != nullptr)
    hipExtLaunchKernelGGL(k_gemm_prefill<1>, dim3(tiles), dim3(NT), 0, s, e0, e1, 0, Xq, Wq, M, N,
                          K, ldk, x_scale, w_scale, XO, WO, n_out, nullptr, Y, C, 0);
  else
    hipExtLaunchKernelGGL(k_gemm_prefill<0>, dim3(tiles + nhalf), dim3(NT), 0, s, e0, e1, 0, Xq,
                          Wq, M, N, K, ldk, x_scale, w_scale, XO, WO, n_out, bias, Y, C, nhalf);
  return hipGetLastError();
}

int gemm_prefill_nhalf(int M, int N, int n_cu) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (n_cu <= 0) return 0;
  // one workgroup per CU: every tile when they fill at most half of the CUs,
  // else the tiles of a last round that fills at most half of them
  if (2 * tiles <= n_cu) return tiles;
  const int tail = tiles % n_cu;
  return tiles >= n_cu && 2 * tail <= n_cu ? tail : 0;
}

}  // namespace i8mm
