// Decode-shaped (M <= 16 rows) decomposed int8 matmul: one streaming pass
// over the int8 weight, which is what bounds it (HBM), with the outlier
// columns handled inline so that Wq is read exactly once per call.
//
// Work split: a workgroup owns G groups of 16 weight rows (output columns n)
// and 8 waves split K between them.  Per 64-byte K step a wave loads one
// 16-byte Xq fragment (rows m = lane%16, zero for m >= M) and G 16-byte Wq
// fragments and issues G v_mfma_i32_16x16x64_i8.  When the 64-column window
// holds an outlier column (wave-uniform test on the mask bits), the wave
// also builds fp16 fragments of X_O (X values of the outlier columns, 0
// elsewhere) and of W_O = fp16(fp32(Wq*a_w)/127) from the int8 bytes already
// in registers, and accumulates them with v_mfma_f32_16x16x32_f16 into
// separate fp32 accumulators ("LLM.int8() notes", section 2.3: FP16 outlier
// term; "PyTorch 2.9 supports LLM.int8()", section 3: merged at the end).
// The 8 per-wave partials are summed in LDS in a fixed order (deterministic)
// and the epilogue writes Y = fp16(fp32(C)*a_x*a_w/127^2 + Y_O).
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

namespace {
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kU = 2;  // K steps per loop iteration
constexpr int kSlots = 8;  // outlier K steps parked in LDS (more: static schedule)
constexpr int kMaxWords = (133144 + 63) / 64 * 2;  // mask words for the largest K
}  // namespace

// A 16-byte Wq fragment.  The weight is read once per call and never again
// in it: nontemporal loads (measured 4.95 -> 5.55 TB/s over the
// 8192 x 28672 weight) keep it from displacing what the caches do reuse.
__device__ __forceinline__ v4i wload(const int8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

template <int G, int MODE>  // MODE 0: Y, 1: int32 C
__global__ __launch_bounds__(kThreads) void k_gemm_decode(
    const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int K, int ldk,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale,
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ mask_bits,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C) {
  __shared__ uint32_t s_bits[kMaxWords];
  __shared__ int s_red[kWaves][G * 256];
  __shared__ v4i s_wslot[kSlots][G][64];  // Wq fragments of the outlier steps
  __shared__ int s_slot_step[kSlots];
  __shared__ int s_nslots;
  __shared__ int s_next;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nw = ldk / 32;
  const int nsteps = ldk / 64;
  if (t == 0) {
    s_nslots = 0;
    s_next = 0;
  }
  __syncthreads();
  for (int w = t; w < nw; w += kThreads) s_bits[w] = mask_bits[w];
  __syncthreads();
  // K steps holding outlier columns, in ascending order (one wave, ballots)
  if (wave == 0) {
    int cnt = 0;
    for (int s0 = 0; s0 < nsteps; s0 += 64) {
      const int st = s0 + lane;
      const bool f = st < nsteps && (s_bits[2 * st] | s_bits[2 * st + 1]) != 0u;
      const uint64_t bal = __ballot(f);
      const int rank = cnt + __popcll(bal & ((1ull << lane) - 1ull));
      if (f && rank < kSlots) s_slot_step[rank] = st;
      cnt += __popcll(bal);
    }
    if (lane == 0) s_nslots = cnt;
  }
  __syncthreads();
  const int n_oslots = s_nslots;
  const bool has_outliers = n_oslots > 0;
  // Few outlier steps: the int8 work is handed out dynamically (the waves of
  // a workgroup finish together instead of the slowest setting the pace) and
  // the outlier steps' Wq fragments are parked in LDS for a fixed-order fp16
  // pass at the end (the result stays deterministic).  Many: static split
  // with the outlier term inline.
  const bool dynamic = n_oslots <= kSlots;

  const int n_base = blockIdx.x * (G * 16);
  const int s0 = (nsteps * wave) / kWaves, s1 = (nsteps * (wave + 1)) / kWaves;
  const int ml = lane & 15;   // row of the Xq fragment / column of the result
  const int kq = (lane >> 4) * 16;  // byte offset of this lane inside the 64-byte step

  // panel-tiled operands (tile_layout.h): step s of row r is at
  // tiled_offset(r, 64*s + kq) = tiled_offset(r, kq) + s * 16 KiB; the 16 rows
  // of a group are 1 KiB contiguous per step
  const int8_t* xrow = Xq + tiled_offset(ml, kq, ldk);
  const bool xvalid = ml < M;
  // The grid covers ceil(groups / G) * G groups of 16 rows, which can run past
  // the prepared weight's padded rows when G does not divide the group count:
  // such groups read the last padded row instead (their results are never
  // stored, n >= N), so every load stays inside the weight.
  const int row_cap = (int)padded_rows(N) - 1;
  const int8_t* wrow[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    wrow[g] = Wq + tiled_offset(min(n_base + g * 16 + ml, row_cap), kq, ldk);

  v4i acc[G];
  v4f acco[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    acc[g] = v4i{};
    acco[g] = v4f{};
  }

  // fp16 outlier term of step s for this lane's 16 columns k0 .. k0+15 (b:
  // the step's Wq fragments, already in registers)
  auto outlier_step = [&](int s, const v4i (&b)[G]) {
    const int k0 = s * 64 + kq;
    const uint32_t ob = (s_bits[k0 >> 5] >> (k0 & 31)) & 0xffffu;
    v8h xa[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      uint16_t v = 0;
      if (((ob >> e) & 1u) && xvalid) v = X[(size_t)ml * K + k0 + e];
      xa[e >> 3][e & 7] = __builtin_bit_cast(_Float16, v);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int n = min(n_base + g * 16 + ml, N - 1);
      const float aw = w_scale[n];
      v8h wb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uint16_t v = 0;
        if ((ob >> e) & 1u) {
          const int q = (int)(int8_t)((b[g][e >> 2] >> ((e & 3) * 8)) & 0xff);
          v = dequant_w_half(q, aw);
        }
        wb[e >> 3][e & 7] = __builtin_bit_cast(_Float16, v);
      }
      acco[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], wb[0], acco[g], 0, 0, 0);
      acco[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], wb[1], acco[g], 0, 0, 0);
    }
  };
  auto step_has_outliers = [&](int s) { return (s_bits[2 * s] | s_bits[2 * s + 1]) != 0u; };

  if (dynamic) {
    // chunks of kU steps from a workgroup counter, fetched one chunk ahead
    int base = 0;
    if (lane == 0) base = atomicAdd(&s_next, kU);
    base = __builtin_amdgcn_readfirstlane(base);
    while (base < nsteps) {
      int nb = 0;
      if (lane == 0) nb = atomicAdd(&s_next, kU);
      v4i b[kU][G];
      v4i a[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int sl = min(base + u, nsteps - 1);  // a short last chunk re-reads, not counted
        const size_t off = (size_t)sl * kTileBytes;
#pragma unroll
        for (int g = 0; g < G; ++g) b[u][g] = wload(wrow[g] + off);
        a[u] = (xvalid && base + u < nsteps) ? *reinterpret_cast<const v4i*>(xrow + off) : v4i{};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g)
          acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][g], acc[g], 0, 0, 0);
      if (has_outliers) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int st = min(base + u, nsteps - 1);
          if (base + u < nsteps && step_has_outliers(st)) {
            int k = 0;
            while (s_slot_step[k] != st) ++k;  // present: at most kSlots entries
#pragma unroll
            for (int g = 0; g < G; ++g) s_wslot[k][g][lane] = b[u][g];
          }
        }
      }
      base = __builtin_amdgcn_readfirstlane(nb);
    }
    __syncthreads();
    // fp16 outlier term, slot k on wave k % kWaves, in slot order
    for (int k = wave; k < n_oslots; k += kWaves) {
      v4i b[G];
#pragma unroll
      for (int g = 0; g < G; ++g) b[g] = s_wslot[k][g][lane];
      outlier_step(s_slot_step[k], b);
    }
  } else {
    // kU steps per iteration: all their loads are issued before the first
    // MFMA, so a wave keeps kU*G KiB of weight reads in flight
    int s = s0;
    for (; s + kU <= s1; s += kU) {
      v4i b[kU][G];
      v4i a[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const size_t off = (size_t)(s + u) * kTileBytes;
#pragma unroll
        for (int g = 0; g < G; ++g) b[u][g] = wload(wrow[g] + off);
        a[u] = xvalid ? *reinterpret_cast<const v4i*>(xrow + off) : v4i{};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g)
          acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][g], acc[g], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (step_has_outliers((s + u))) outlier_step((s + u), b[u]);
    }
    for (; s < s1; ++s) {
      const size_t off = (size_t)s * kTileBytes;
      v4i b[G];
#pragma unroll
      for (int g = 0; g < G; ++g) b[g] = wload(wrow[g] + off);
      const v4i a = xvalid ? *reinterpret_cast<const v4i*>(xrow + off) : v4i{};
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[g], acc[g], 0, 0, 0);
      if (step_has_outliers(s)) outlier_step(s, b);
    }
  }

  // ---- fixed-order reduction of the 8 wave partials.  Element e = g*256 +
  // lane*4 + r of a wave holds result row m = 4*(lane/16) + r, column
  // n = n_base + 16*g + lane%16 (16x16 MFMA accumulator layout).
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[wave][g * 256 + lane * 4 + r] = acc[g][r];
  __syncthreads();
  int csum[(G * 256 + kThreads - 1) / kThreads];
#pragma unroll
  for (int u = 0; u < (G * 256 + kThreads - 1) / kThreads; ++u) {
    const int e = t + u * kThreads;
    int v = 0;
    if (e < G * 256) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += s_red[w][e];
    }
    csum[u] = v;
  }
  float osum[(G * 256 + kThreads - 1) / kThreads];
#pragma unroll
  for (int u = 0; u < (G * 256 + kThreads - 1) / kThreads; ++u) osum[u] = 0.0f;
  if (MODE == 0 && has_outliers) {
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_red[wave][g * 256 + lane * 4 + r] = __float_as_int(acco[g][r]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (G * 256 + kThreads - 1) / kThreads; ++u) {
      const int e = t + u * kThreads;
      float v = 0.0f;
      if (e < G * 256) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += __int_as_float(s_red[w][e]);
      }
      osum[u] = v;
    }
  }
#pragma unroll
  for (int u = 0; u < (G * 256 + kThreads - 1) / kThreads; ++u) {
    const int e = t + u * kThreads;
    if (e >= G * 256) continue;
    const int g = e >> 8, ln = (e >> 2) & 63, r = e & 3;
    const int m = (ln >> 4) * 4 + r;
    const int n = n_base + g * 16 + (ln & 15);
    if (m >= M || n >= N) continue;
    if (MODE == 1) {
      C[(size_t)m * N + n] = csum[u];
    } else {
      const float sc = x_scale[m] * w_scale[n] * kInv127Sq;
      const float b = bias != nullptr ? h2f(bias[n]) : 0.0f;
      Y[(size_t)m * N + n] = f2h((float)csum[u] * sc + osum[u] + b);
    }
  }
}

template <int G>
static void launch_g(dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const int8_t* Xq, const int8_t* Wq, int M, int N,
                     int K, int ldk, const float* xs, const float* ws, const uint16_t* X,
                     const uint32_t* mb, const uint16_t* bias, uint16_t* Y, int32_t* C) {
  if (C != nullptr)
    hipExtLaunchKernelGGL((k_gemm_decode<G, 1>), grid, dim3(kThreads), 0, s, e0, e1, 0, Xq, Wq, M,
                          N, K, ldk, xs, ws, X, mb, bias, Y, C);
  else
    hipExtLaunchKernelGGL((k_gemm_decode<G, 0>), grid, dim3(kThreads), 0, s, e0, e1, 0, Xq, Wq, M,
                          N, K, ldk, xs, ws, X, mb, bias, Y, C);
}

hipError_t launch_gemm_decode(const int8_t* Xq, const int8_t* Wq, int M, int N, int K, int ldk,
                              const float* x_scale, const float* w_scale, const uint16_t* X,
                              const uint32_t* mask_bits, const uint16_t* bias, uint16_t* Y,
                              int32_t* C, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  // Spread the 16-row groups evenly over the 256 CUs: G groups per workgroup.
  const int groups = (N + 15) / 16;
  int G = (groups + 255) / 256;
  if (G > 8) G = 8;
  if (G < 1) G = 1;
  dim3 grid((groups + G - 1) / G);
  switch (G) {
    case 1: launch_g<1>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
    case 2: launch_g<2>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
    case 3: launch_g<3>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
    case 4: launch_g<4>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
    case 5: launch_g<5>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
    case 6: launch_g<6>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
    case 7: launch_g<7>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
    default: launch_g<8>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, bias, Y, C); break;
  }
  return hipGetLastError();
}

}  // namespace i8mm
