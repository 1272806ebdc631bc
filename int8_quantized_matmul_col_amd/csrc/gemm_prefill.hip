// Prefill GEMM of the decomposed int8 matmul on gfx950 matrix cores.
//
//   Y[m,n] = fp16( fp32(C[m,n]) * a_x[m]*a_w[n]/127^2 + sum_j X_O[m,j] W_O[n,j] )
//   C[m,n] = sum_k Xq[m,k] Wq[n,k]                         (int32, exact)
//
// ("LLM.int8() notes", section 2.3: the INT8 term plus the FP16 outlier term;
// "PyTorch 2.9 supports LLM.int8()", section 3: results merged at the end.)
//
// One workgroup = 256x256 output tile, 4 waves in a 2x2 arrangement, each
// wave a 128x128 block held as 4x4 v_mfma_i32_32x32x32_i8 accumulators
// (256 AGPRs).  Operands are panel-tiled in memory (tile_layout.h), so one
// 64-byte K step of a 256-row panel is 16 KiB contiguous: every wave load
// instruction moves 1 KiB of whole cache lines straight into LDS
// (global_load_lds_dwordx4: no VGPR staging, no ds_write).  Four LDS stages
// let loads run two steps ahead and let the first fragments of step k+1 be
// read before the barrier that ends step k; one barrier per step.
//
// The outlier slice (|O| rounded up to 32 fp16 columns: 64 bytes per row per
// step, the same byte shape as an int8 step) is appended to the same
// pipeline as extra steps on v_mfma_f32_32x32x16_f16: their loads are issued
// during the last int8 steps, the int32 accumulators are rescaled to fp32 in
// place in between, and the fp16 products accumulate on top.  |O| is read on
// the device: no host synchronisation.
//
// MFMA operand convention: lane l supplies row (l%32) of its operand and 16
// bytes of K; A and B fragments use the same K mapping, so the pairing of K
// indices is consistent whatever order the hardware assigns inside the 16
// bytes (exact for the int8 sum, within fp32 rounding for fp16).
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

namespace {

constexpr int BM = kPanelRows;  // 256
constexpr int BN = kPanelRows;
constexpr int NT = 256;
constexpr int NBUF = 4;  // LDS stages of 256 rows x 64 bytes per operand

struct Smem {
  v4i a[NBUF][BM * 4];
  v4i b[NBUF][BN * 4];
  float sx[BM];
  float sw[BN];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS slot of 16-byte chunk `ch` (0..3) of tile row `row`.  gfx950 LDS serves
// a 16-byte read in groups of 16 lanes (64 banks, 256 B/clk): 16 consecutive
// rows then hit 16 distinct slots when the chunk is XORed with bits 2..3 of
// the row.  The direct-to-LDS loads fill 64 consecutive slots per wave
// instruction, so the swizzle is applied on the global-address side.
__device__ __forceinline__ int swz(int row, int ch) { return row * 4 + (ch ^ ((row >> 2) & 3)); }

// Source of pipeline step s: int8 steps first, then fp16 outlier steps.
struct Src {
  const char* A;  // panel-tiled; the tile's panel already applied
  const char* B;
  const char* AO;
  const char* BO;
  int nk8;  // number of int8 steps
};

// Issue the loads of step s into stage `buf`: 4 instructions per operand per
// wave, each 64 lanes x 16 bytes = a 1 KiB slice of the 16 KiB block.
__device__ __forceinline__ void gload(Smem& sm, int buf, const Src& src, int s, int wave,
                                      int lane) {
  const char* a;
  const char* b;
  if (s < src.nk8) {
    a = src.A + (size_t)s * kTileBytes;
    b = src.B + (size_t)s * kTileBytes;
  } else {
    a = src.AO + (size_t)(s - src.nk8) * kTileBytes;
    b = src.BO + (size_t)(s - src.nk8) * kTileBytes;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s0 = (i * 4 + wave) * 64;
    const int slot = s0 + lane;
    const int row = slot >> 2;
    const int ch = (slot & 3) ^ ((row >> 2) & 3);
    const int off = row * 64 + ch * 16;
    __builtin_amdgcn_global_load_lds((const void*)(a + off), (lds_ptr_t)&sm.a[buf][s0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(b + off), (lds_ptr_t)&sm.b[buf][s0], 16, 0, 0);
  }
}

// MFMA operand fragments of one 32-byte K sub-step for the wave's 4x4 tiles.
struct Frag {
  v4i a[4];
  v4i b[4];
};

__device__ __forceinline__ void fload(Frag& f, const Smem& sm, int buf, int kk, int wm0, int wn0,
                                      int lane) {
  const int ch = kk * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = sm.a[buf][swz(wm0 + i * 32 + (lane & 31), ch)];
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = sm.b[buf][swz(wn0 + j * 32 + (lane & 31), ch)];
}

template <bool F16>
__device__ __forceinline__ void mma(const Frag& f, v16i (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (F16) {
        // acc holds fp32 bit patterns here (reinterpreted in place)
        acc[i][j] = __builtin_bit_cast(
            v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, f.a[i]),
                                                         __builtin_bit_cast(v8h, f.b[j]),
                                                         __builtin_bit_cast(v16f, acc[i][j]), 0,
                                                         0, 0));
      } else {
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
      }
    }
}

// s_waitcnt: vmcnt <= 8 (the loads issued in the current step may stay in
// flight) and lgkmcnt 0; or everything.
__device__ __forceinline__ void wait_prev_step() {
  __builtin_amdgcn_s_waitcnt((8 & 0xf) | (7 << 4) | (0 << 8) | ((8 >> 4) << 14));
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// One pipeline step: fragments of sub-step 1 while sub-step 0 computes, the
// next step's sub-step-0 fragments while sub-step 1 computes, the loads of
// step kt+3; then wait for the loads of step kt+2 and this wave's LDS reads,
// and the barrier.  Branch-free: loads past the end are clamped to the last
// step (in bounds, landing in a stage that is not read again).
template <bool F16>
__device__ __forceinline__ void step(Smem& sm, v16i (&acc)[4][4], Frag& f0, Frag& f1,
                                     const Src& src, int kt, int last, int wm0, int wn0, int wave,
                                     int lane) {
  const int cur = kt & 3, nxt = (kt + 1) & 3, far = (kt + 3) & 3;
  fload(f1, sm, cur, 1, wm0, wn0, lane);
  mma<F16>(f0, acc);
  fload(f0, sm, nxt, 0, wm0, wn0, lane);
  mma<F16>(f1, acc);
  gload(sm, far, src, min(kt + 3, last), wave, lane);
  // sub-step-1 reads over the first 8 MFMAs, prefetch reads over the third
  // group of 8, the 8 global loads over the last 8 MFMAs
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
  }
  wait_prev_step();
  __builtin_amdgcn_s_barrier();
}

// Row (within the wave block) of accumulator element r of lane `lane` for a
// 32x32 MFMA tile: rows 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

}  // namespace

// Many outlier columns (more than three fp16 steps): dequantize the int32
// accumulators in place and continue the pipeline over the fp16 steps on
// top.  Kept out of line so that its register pressure does not shape the
// common path's allocation; it recomputes the whole tile.
__device__ __attribute__((noinline)) void gemm_tile_many_outliers(
    Smem& sm, const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int ldk,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale,
    const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
    const int32_t* __restrict__ n_out, uint16_t* __restrict__ Y, int32_t* __restrict__ C) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;

  // XCD-aware tile order: consecutive workgroups go round-robin to the 8
  // XCDs, so give each XCD a contiguous run of tiles, and walk the tiles in
  // groups of 4 tile-rows so the run shares A and B panels in its L2.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int G = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int L = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  constexpr int GROUP = 4;
  const int per_group = GROUP * tiles_n;
  const int first_m = (L / per_group) * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (L % per_group) % gsz;
  const int tn = (L % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

  const int nk8 = ldk / kTileK;
  const int nk16 = (*n_out + 31) / 32;
  const int last = nk8 + nk16 - 1;
  Src src;
  src.A = (const char*)Xq + (size_t)tm * nk8 * kTileBytes;
  src.B = (const char*)Wq + (size_t)tn * nk8 * kTileBytes;
  src.AO = (const char*)XO + (size_t)tm * (2 * nk8) * kTileBytes;  // fp16 rows: 2*ldk bytes
  src.BO = (const char*)WO + (size_t)tn * (2 * nk8) * kTileBytes;
  src.nk8 = nk8;

  // prologue: stages 0..2
  gload(sm, 0, src, 0, wave, lane);
  gload(sm, 1, src, min(1, last), wave, lane);
  gload(sm, 2, src, min(2, last), wave, lane);
  wait_all();
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
  fload(f0, sm, 0, 0, wm0, wn0, lane);

  // ---- int8 x int8 -> int32 over all K (outlier columns of Xq are zero)
  int kt = 0;
  for (; kt < nk8; ++kt) step<false>(sm, acc, f0, f1, src, kt, last, wm0, wn0, wave, lane);

  if (false) {
    wait_all();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm0 + i * 32 + acc_row(r, lane);
          const int n = n0 + wn0 + j * 32 + (lane & 31);
          if (m < M && n < N) C[(size_t)m * N + n] = acc[i][j][r];
        }
    return;
  }

  // ---- scales of the tile's rows and columns
  {
    const int t = threadIdx.x;
    sm.sx[t] = x_scale[min(m0 + t, M - 1)];
    sm.sw[t] = w_scale[min(n0 + t, N - 1)] * kInv127Sq;
  }
  const int n_col = n0 + wn0 + (lane & 15) * 8;
  const bool vec_store = (N & 7) == 0;

  // ---- many outlier columns: dequantize in place, fp32(C) * a_x[m] * a_w[n]
  // / 127^2, and continue the pipeline over the fp16 steps on top.
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float sx[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f v = *reinterpret_cast<const v4f*>(&sm.sx[wm0 + i * 32 + q * 8 + (lane >> 5) * 4]);
      sx[q * 4 + 0] = v[0];
      sx[q * 4 + 1] = v[1];
      sx[q * 4 + 2] = v[2];
      sx[q * 4 + 3] = v[3];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sw = sm.sw[wn0 + j * 32 + (lane & 31)];
      v16f f;
#pragma unroll
      for (int r = 0; r < 16; ++r) f[r] = (float)acc[i][j][r] * (sx[r] * sw);
      acc[i][j] = __builtin_bit_cast(v16i, f);
    }
  }
  for (; kt <= last; ++kt) step<true>(sm, acc, f0, f1, src, kt, last, wm0, wn0, wave, lane);

  // store fp16 Y through LDS: two 64-row halves per wave, 16 KiB each
  wait_all();
  __syncthreads();
  uint16_t* ys = reinterpret_cast<uint16_t*>(&sm.a[0][0]) + wave * (64 * 128);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = half * 2 + ii;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v16f f = __builtin_bit_cast(v16f, acc[i][j]);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ys[(ii * 32 + acc_row(r, lane)) * 128 + j * 32 + (lane & 31)] = f2h(f[r]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int rl = p * 4 + (lane >> 4);  // row within the 64-row half
      const int m = m0 + wm0 + half * 64 + rl;
      const v4i v = *reinterpret_cast<const v4i*>(ys + rl * 128 + (lane & 15) * 8);
      if (m < M) {
        if (vec_store && n_col + 8 <= N) {
          *reinterpret_cast<v4i*>(Y + (size_t)m * N + n_col) = v;
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
}


template <int MODE>  // 0: Y (fused epilogue), 1: int32 C
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void
k_gemm_prefill(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int ldk,
               const float* __restrict__ x_scale, const float* __restrict__ w_scale,
               const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
               const int32_t* __restrict__ n_out, uint16_t* __restrict__ Y,
               int32_t* __restrict__ C) {
  __shared__ Smem sm;
  if (MODE == 0 && (*n_out + 31) / 32 > 3) {
    gemm_tile_many_outliers(sm, Xq, Wq, M, N, ldk, x_scale, w_scale, XO, WO, n_out, Y, C);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;

  // XCD-aware tile order: consecutive workgroups go round-robin to the 8
  // XCDs, so give each XCD a contiguous run of tiles, and walk the tiles in
  // groups of 4 tile-rows so the run shares A and B panels in its L2.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int G = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int L = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  constexpr int GROUP = 4;
  const int per_group = GROUP * tiles_n;
  const int first_m = (L / per_group) * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (L % per_group) % gsz;
  const int tn = (L % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  v16i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

  const int nk8 = ldk / kTileK;
  const int nk16 = MODE == 0 ? (*n_out + 31) / 32 : 0;
  const int last = nk8 + nk16 - 1;
  Src src;
  src.A = (const char*)Xq + (size_t)tm * nk8 * kTileBytes;
  src.B = (const char*)Wq + (size_t)tn * nk8 * kTileBytes;
  src.AO = (const char*)XO + (size_t)tm * (2 * nk8) * kTileBytes;  // fp16 rows: 2*ldk bytes
  src.BO = (const char*)WO + (size_t)tn * (2 * nk8) * kTileBytes;
  src.nk8 = nk8;

  // prologue: stages 0..2
  gload(sm, 0, src, 0, wave, lane);
  gload(sm, 1, src, min(1, last), wave, lane);
  gload(sm, 2, src, min(2, last), wave, lane);
  wait_all();
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
  fload(f0, sm, 0, 0, wm0, wn0, lane);

  // ---- int8 x int8 -> int32 over all K (outlier columns of Xq are zero)
  int kt = 0;
  for (; kt < nk8; ++kt) step<false>(sm, acc, f0, f1, src, kt, last, wm0, wn0, wave, lane);

  if (MODE == 1) {
    wait_all();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm0 + i * 32 + acc_row(r, lane);
          const int n = n0 + wn0 + j * 32 + (lane & 31);
          if (m < M && n < N) C[(size_t)m * N + n] = acc[i][j][r];
        }
    return;
  }

  // ---- scales of the tile's rows and columns
  {
    const int t = threadIdx.x;
    sm.sx[t] = x_scale[min(m0 + t, M - 1)];
    sm.sw[t] = w_scale[min(n0 + t, N - 1)] * kInv127Sq;
  }
  const int n_col = n0 + wn0 + (lane & 15) * 8;
  const bool vec_store = (N & 7) == 0;

  {
    // Few outlier steps: their operands were prefetched into LDS stages
    // (nk8 + s) & 3 by the int8 loop.  Per 32-row group i: the outlier
    // product into a 64-register temporary, then Y = fp32(C)*s + Y_O read
    // straight from the int32 accumulators, converted to fp16, staged in the
    // free LDS stage (nk8 + 3) & 3 (8 KiB per wave) and stored as 256-byte
    // row segments.
    wait_all();
    __syncthreads();
    const int fs = (nk8 + 3) & 3;
    uint16_t* ys = reinterpret_cast<uint16_t*>(wave < 2 ? &sm.a[fs][0] : &sm.b[fs][0]) +
                   (wave & 1) * (32 * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // row group i: scaled int8 part first (its accumulator registers are
      // then free for the fp16 MFMAs), outlier products accumulated on top
      float sx[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f v =
            *reinterpret_cast<const v4f*>(&sm.sx[wm0 + i * 32 + q * 8 + (lane >> 5) * 4]);
        sx[q * 4 + 0] = v[0];
        sx[q * 4 + 1] = v[1];
        sx[q * 4 + 2] = v[2];
        sx[q * 4 + 3] = v[3];
      }
      v16f y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sw = sm.sw[wn0 + j * 32 + (lane & 31)];
#pragma unroll
        for (int r = 0; r < 16; ++r) y[j][r] = (float)acc[i][j][r] * (sx[r] * sw);
      }
      for (int st = 0; st < nk16; ++st) {
        const int stg = (nk8 + st) & 3;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ch = kk * 2 + (lane >> 5);
          const v8h a = __builtin_bit_cast(v8h, sm.a[stg][swz(wm0 + i * 32 + (lane & 31), ch)]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v8h b = __builtin_bit_cast(v8h, sm.b[stg][swz(wn0 + j * 32 + (lane & 31), ch)]);
            y[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, y[j], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ys[acc_row(r, lane) * 128 + j * 32 + (lane & 31)] = f2h(y[j][r]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int rl = p * 4 + (lane >> 4);  // row within the 32-row group
        const int m = m0 + wm0 + i * 32 + rl;
        const v4i v = *reinterpret_cast<const v4i*>(ys + rl * 128 + (lane & 15) * 8);
        if (m < M) {
          if (vec_store && n_col + 8 <= N) {
            *reinterpret_cast<v4i*>(Y + (size_t)m * N + n_col) = v;
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
    return;
  }

}

hipError_t launch_gemm_prefill(const int8_t* Xq, const int8_t* Wq, int M, int N, int ldk,
                               const float* x_scale, const float* w_scale, const uint16_t* XO,
                               const uint16_t* WO, const int32_t* n_out, uint16_t* Y, int32_t* C,
                               hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (C != nullptr)
    hipExtLaunchKernelGGL(k_gemm_prefill<1>, dim3(tiles), dim3(NT), 0, s, e0, e1, 0, Xq, Wq, M, N,
                          ldk, x_scale, w_scale, XO, WO, n_out, Y, C);
  else
    hipExtLaunchKernelGGL(k_gemm_prefill<0>, dim3(tiles), dim3(NT), 0, s, e0, e1, 0, Xq, Wq, M, N,
                          ldk, x_scale, w_scale, XO, WO, n_out, Y, C);
  return hipGetLastError();
}

}  // namespace i8mm
