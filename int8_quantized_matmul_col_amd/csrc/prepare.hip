// One-time per-output-channel weight quantization ("PyTorch 2.9 supports
// LLM.int8()", section 1: one absmax/127 scale per output channel, weights
// rounded to int8 once, before the first inference).
//
// Rows up to 32768 columns (every shape of the workloads): one workgroup of
// 8 waves per 4 weight rows reads each row once, into registers, in the
// arrangement of its stores: lane l holds row (l/4) mod 4, 16 columns of
// column block 4*(wave + 8*j) + l/16 for j < J, so that one store instruction
// of a wave writes four whole 256-byte pieces of the panel-tiled layout
// (4 rows x 64 bytes of a column block are contiguous there) and the loads of
// 4 lanes cover whole 128-byte lines of a row.  The row absmax is reduced
// across the lanes of a row in a wave and then across the waves through LDS.
// The codes use the fast reciprocal form with the IEEE-division fallback near
// rounding ties (bit-identical to the division for every binary16 pair); rows
// past N (the padding of the last panel) and columns past K are written as
// zeros.  (Measured on MI355X against 8 and 2 rows per workgroup: 4 was the
// fastest or within 15% of it on every weight shape of the workloads.)
//
// Longer rows: one wave per row, two passes (max |W[n,:]|, then the codes
// from a re-read of the row, 8 at a time).
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

namespace {
constexpr int kPrepRows = 4;    // weight rows per workgroup (register form)
constexpr int kPrepWaves = 8;   // waves per workgroup (register form)
constexpr int kPrepMaxJ = 16;   // load rounds held in registers
}  // namespace

template <int ROWS, int J>
__global__ __launch_bounds__(kPrepWaves * 64) void k_prepare_weight_regs(
    const uint16_t* __restrict__ W, int N, int K, int ldk, int vec, int8_t* __restrict__ Wq,
    float* __restrict__ w_scale) {
  constexpr int kBW = 64 / (4 * ROWS);       // column blocks per wave instruction
  constexpr int kBlocks = kBW * kPrepWaves;  // column blocks per load round
  __shared__ uint32_t s_m[kPrepWaves][ROWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = (lane >> 2) % ROWS;
  const int n = blockIdx.x * ROWS + rr;
  const bool live = n < N;
  const uint16_t* row = W + (size_t)min(n, N - 1) * K;
  const int nb = ldk / 64;
  const int cb0 = kBW * wave + lane / (4 * ROWS);
  const int cofs = (lane & 3) * 16;

  uint4 w[J][2];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int cb = cb0 + j * kBlocks;
    if (live && cb < nb) {
      w[j][0] = load_chunk(row, cb * 64 + cofs, K, vec != 0);
      w[j][1] = load_chunk(row, cb * 64 + cofs + 8, K, vec != 0);
    } else {
      w[j][0] = uint4{0u, 0u, 0u, 0u};
      w[j][1] = uint4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t m2 = 0;  // two packed 16-bit |x| maxima
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4& v = w[j][h];
      m2 = pk_max_u16(m2, pk_max_u16(pk_max_u16(v.x & 0x7fff7fffu, v.y & 0x7fff7fffu),
                                     pk_max_u16(v.z & 0x7fff7fffu, v.w & 0x7fff7fffu)));
    }
  uint32_t mx = max(m2 & 0xffffu, m2 >> 16);
  // the lanes of row rr in this wave: rr*4 + {0..3} in each group of 4*ROWS
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, 64));
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, 64));
#pragma unroll
  for (int o = 4 * ROWS; o < 64; o *= 2) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if (lane < 4 * ROWS && (lane & 3) == 0) s_m[wave][rr] = mx;
  __syncthreads();
  uint32_t am = 0;
#pragma unroll
  for (int v = 0; v < kPrepWaves; ++v) am = max(am, s_m[v][rr]);
  const float a = h2f((uint16_t)am);
  if (wave == 0 && lane < 4 * ROWS && (lane & 3) == 0 && live) w_scale[n] = a;
  const float r = a == 0.0f ? 0.0f : 127.0f / a;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int cb = cb0 + j * kBlocks;
    if (cb < nb) {
      float d0, d1;
      uint2 q0 = quant8_fast(w[j][0], r, &d0);
      uint2 q1 = quant8_fast(w[j][1], r, &d1);
      if (d0 > kTieGuard) q0 = quant8_exact(w[j][0], a);
      if (d1 > kTieGuard) q1 = quant8_exact(w[j][1], a);
      *reinterpret_cast<uint4*>(Wq + tiled_offset(n, (size_t)(cb * 64 + cofs), ldk)) =
          uint4{q0.x, q0.y, q1.x, q1.y};
    }
  }
}

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

template <int ROWS>
static bool launch_regs(const uint16_t* W, int N, int K, int ldk, int vec, int8_t* Wq,
                        float* w_scale, hipStream_t s) {
  constexpr int kBlocks = 64 / (4 * ROWS) * kPrepWaves;
  const int rounds = (ldk / 64 + kBlocks - 1) / kBlocks;
  if (rounds > kPrepMaxJ) return false;
  const dim3 grid((unsigned)(padded_rows(N) / ROWS)), block(kPrepWaves * 64);
#define PREP(J) \
  hipLaunchKernelGGL((k_prepare_weight_regs<ROWS, J>), grid, block, 0, s, W, N, K, ldk, vec, Wq, w_scale)
  if (rounds <= 1) PREP(1);
  else if (rounds <= 2) PREP(2);
  else if (rounds <= 4) PREP(4);
  else if (rounds <= 8) PREP(8);
  else PREP(16);
#undef PREP
  return true;
}

// ---------------------------------------------------------------- packing

// Already-quantized weights ("PyTorch 2.9 supports LLM.int8()", section 1: the
// stored 8-bit weight is its int8 codes plus one scale per output channel):
// row-major [N][K] codes into the panel-tiled layout, codes clamped to
// [-127, 127], padding rows and columns zero.  A wave fills one 64-byte
// column block of 16 consecutive rows, which is 1 KiB contiguous in the tiled
// layout (lane l: row r0 + l/4, bytes 16*(l%4) .. +15 of the block).
__global__ __launch_bounds__(256) void k_pack_weight(const int8_t* __restrict__ src, int N, int K,
                                                     int ldk, int vec, int8_t* __restrict__ Wq) {
  const int lane = threadIdx.x & 63;
  const int nblk = ldk / 64;
  const long g = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (16-row group, block) index
  const int rg = (int)(g / nblk), b = (int)(g % nblk);
  const int n = rg * 16 + (lane >> 2);
  const int k0 = b * 64 + (lane & 3) * 16;
  if (n >= (int)padded_rows(N)) return;
  int8_t v[16];
  if (n < N && vec && k0 + 16 <= K) {
    const int4 w = *reinterpret_cast<const int4*>(src + (size_t)n * K + k0);
    __builtin_memcpy(v, &w, 16);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = (n < N && k0 + e < K) ? src[(size_t)n * K + k0 + e] : 0;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = v[e] < -kQMax ? (int8_t)-kQMax : v[e];
  int4 o;
  __builtin_memcpy(&o, v, 16);
  *reinterpret_cast<int4*>(Wq + tiled_offset(n, (size_t)k0, ldk)) = o;
}

hipError_t launch_pack_weight(const int8_t* src, int N, int K, int ldk, int8_t* Wq,
                              hipStream_t s) {
  const int vec = (K % 16 == 0) && ((reinterpret_cast<uintptr_t>(src) & 15) == 0);
  const long waves = (long)(padded_rows(N) / 16) * (ldk / 64);
  hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, src, N, K,
                     ldk, vec, Wq);
  return hipGetLastError();
}

hipError_t launch_prepare_weight(const uint16_t* W, int N, int K, int ldk, int8_t* Wq,
                                 float* w_scale, hipStream_t s) {
  const int vec = (K % 8 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
  if (!launch_regs<kPrepRows>(W, N, K, ldk, vec, Wq, w_scale, s)) {
    const dim3 grid((unsigned)(padded_rows(N) / 4));
    hipLaunchKernelGGL(k_prepare_weight, grid, dim3(256), 0, s, W, N, K, ldk, vec, Wq, w_scale);
  }
  return hipGetLastError();
}

}  // namespace i8mm
