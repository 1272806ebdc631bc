// Prefill GEMM of the decomposed int8 matmul on gfx950 matrix cores.
//
//   Y[m,n] = fp16( fp32(C[m,n]) * a_x[m]*a_w[n]/127^2 + sum_j X_O[m,j] W_O[n,j] )
//   C[m,n] = sum_k Xq[m,k] Wq[n,k]                         (int32, exact)
//
// ("LLM.int8() notes", section 2.3: the INT8 term plus the FP16 outlier term;
// "PyTorch 2.9 supports LLM.int8()", section 3: results merged at the end.)
//
// One workgroup = 256x256 output tile, 4 waves in a 2x2 arrangement, each
// wave a 128x128 block held as 4x4 v_mfma_i32_32x32x32_i8 accumulators.  The
// K loop stages 64-byte slices of Xq and Wq through double-buffered LDS
// (one barrier per step); 16-byte chunks are XOR-swizzled so that both the
// 16-byte stores and the ds_read_b128 fragment reads are bank-conflict free.
// After the int8 loop the accumulators are rescaled to fp32 in place and the
// outlier slice (|O| rounded up to 32 columns of fp16) runs through the same
// pipeline on v_mfma_f32_32x32x16_f16, accumulating on top -- a 64-byte fp16
// slice has exactly the byte layout of a 64-byte int8 slice, so the staging
// and fragment code is shared.  |O| is read on the device: no host sync.
//
// MFMA operand convention: for both instructions lane l supplies row (l%32)
// of its operand and 16 bytes of K; A and B fragments are loaded with the
// same K mapping, so the pairing of K indices is consistent whatever order
// the hardware assigns inside the 16 bytes (the sum over K is order-free
// for the exact int8 product and within fp32 rounding for fp16).
#include "device_common.h"
#include "launch.h"

namespace i8mm {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BKB = 64;  // bytes of K per pipeline step
constexpr int NT = 256;

struct Smem {
  v4i a[2][BM * 4];
  v4i b[2][BN * 4];
  float sx[BM];
  float sw[BN];
};

__device__ __forceinline__ int swz(int row, int ch) { return row * 4 + (ch ^ ((row >> 1) & 3)); }

struct Stage {
  v4i a[4];
  v4i b[4];
};

// Global -> registers for one 64-byte K step.  Rows past the matrix end are
// clamped to the last row (their results are never stored).
__device__ __forceinline__ void gload(Stage& st, const char* __restrict__ A, size_t lda, int a_last,
                                      int m0, const char* __restrict__ B, size_t ldb, int b_last,
                                      int n0, size_t kbyte) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + NT * i;
    const int row = c >> 2, ch = c & 3;
    const int ra = min(m0 + row, a_last);
    const int rb = min(n0 + row, b_last);
    st.a[i] = *reinterpret_cast<const v4i*>(A + (size_t)ra * lda + kbyte + ch * 16);
    st.b[i] = *reinterpret_cast<const v4i*>(B + (size_t)rb * ldb + kbyte + ch * 16);
  }
}

__device__ __forceinline__ void sstore(Smem& sm, int buf, const Stage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + NT * i;
    const int row = c >> 2, ch = c & 3;
    sm.a[buf][swz(row, ch)] = st.a[i];
    sm.b[buf][swz(row, ch)] = st.b[i];
  }
}

__device__ __forceinline__ void mma_i8(const Smem& sm, int buf, int wm0, int wn0, int lane,
                                       v16i (&acc)[4][4]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int ch = kk * 2 + (lane >> 5);
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = sm.a[buf][swz(wm0 + i * 32 + (lane & 31), ch)];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = sm.b[buf][swz(wn0 + j * 32 + (lane & 31), ch)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// acc holds fp32 bit patterns here (reinterpreted in place, no second set
// of 256 accumulator registers).
__device__ __forceinline__ void mma_f16(const Smem& sm, int buf, int wm0, int wn0, int lane,
                                        v16i (&acc)[4][4]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int ch = kk * 2 + (lane >> 5);
    v8h a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = __builtin_bit_cast(v8h, sm.a[buf][swz(wm0 + i * 32 + (lane & 31), ch)]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = __builtin_bit_cast(v8h, sm.b[buf][swz(wn0 + j * 32 + (lane & 31), ch)]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_bit_cast(
            v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j],
                                                         __builtin_bit_cast(v16f, acc[i][j]), 0, 0, 0));
  }
}

// Row (within the wave block) of accumulator element r of lane `lane` for a
// 32x32 MFMA tile: rows 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

}  // namespace

template <int MODE>  // 0: Y (fused epilogue), 1: int32 C
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1))) void
k_gemm_prefill(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int ldk,
               const float* __restrict__ x_scale, const float* __restrict__ w_scale,
               const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
               const int32_t* __restrict__ n_out, uint16_t* __restrict__ Y,
               int32_t* __restrict__ C) {
  __shared__ Smem sm;
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

  // ---- int8 x int8 -> int32 over all K (outlier columns of Xq are zero)
  const int nk = ldk / BKB;
  {
    Stage st;
    gload(st, (const char*)Xq, ldk, M - 1, m0, (const char*)Wq, ldk, N - 1, n0, 0);
    sstore(sm, 0, st);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk)
        gload(st, (const char*)Xq, ldk, M - 1, m0, (const char*)Wq, ldk, N - 1, n0,
              (size_t)(kt + 1) * BKB);
      mma_i8(sm, kt & 1, wm0, wn0, lane, acc);
      if (kt + 1 < nk) sstore(sm, (kt + 1) & 1, st);
      __syncthreads();
    }
  }

  if (MODE == 1) {
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

  // ---- dequantize in place: fp32(C) * a_x[m] * a_w[n] / 127^2
  {
    const int t = threadIdx.x;
    sm.sx[t] = x_scale[min(m0 + t, M - 1)];
    sm.sw[t] = w_scale[min(n0 + t, N - 1)];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sw = sm.sw[wn0 + j * 32 + (lane & 31)] * kInv127Sq;
      v16f f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        f[r] = (float)acc[i][j][r] * (sm.sx[wm0 + i * 32 + acc_row(r, lane)] * sw);
      acc[i][j] = __builtin_bit_cast(v16i, f);
    }

  // ---- fp16 outlier slice: X_O [M][ldk] . W_O [N][ldk]^T over ceil(|O|/32) steps
  const int n_steps = (*n_out + 31) / 32;
  if (n_steps > 0) {
    const size_t ldo = (size_t)ldk * 2;  // bytes per row of X_O / W_O
    Stage st;
    gload(st, (const char*)XO, ldo, M - 1, m0, (const char*)WO, ldo, N - 1, n0, 0);
    sstore(sm, 0, st);
    __syncthreads();
    for (int ks = 0; ks < n_steps; ++ks) {
      if (ks + 1 < n_steps)
        gload(st, (const char*)XO, ldo, M - 1, m0, (const char*)WO, ldo, N - 1, n0,
              (size_t)(ks + 1) * BKB);
      mma_f16(sm, ks & 1, wm0, wn0, lane, acc);
      if (ks + 1 < n_steps) sstore(sm, (ks + 1) & 1, st);
      __syncthreads();
    }
  }

  // ---- store fp16 Y
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm0 + i * 32 + acc_row(r, lane);
        const int n = n0 + wn0 + j * 32 + (lane & 31);
        if (m < M && n < N) Y[(size_t)m * N + n] = f2h(__builtin_bit_cast(v16f, acc[i][j])[r]);
      }
}

hipError_t launch_gemm_prefill(const int8_t* Xq, const int8_t* Wq, int M, int N, int ldk,
                               const float* x_scale, const float* w_scale, const uint16_t* XO,
                               const uint16_t* WO, const int32_t* n_out, uint16_t* Y, int32_t* C,
                               hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (C != nullptr)
    hipLaunchKernelGGL(k_gemm_prefill<1>, dim3(tiles), dim3(NT), 0, s, Xq, Wq, M, N, ldk, x_scale,
                       w_scale, XO, WO, n_out, Y, C);
  else
    hipLaunchKernelGGL(k_gemm_prefill<0>, dim3(tiles), dim3(NT), 0, s, Xq, Wq, M, N, ldk, x_scale,
                       w_scale, XO, WO, n_out, Y, C);
  return hipGetLastError();
}

}  // namespace i8mm
