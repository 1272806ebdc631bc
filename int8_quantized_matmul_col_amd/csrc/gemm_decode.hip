// Decode-shaped (M <= 16 rows) decomposed int8 matmul: one streaming pass
// over the int8 weight, which is what bounds it (HBM), with the outlier
// columns handled inline so that Wq is read exactly once per call.
//
// Work split: a workgroup owns G groups of 16 weight rows (output columns n)
// and 8 waves split K between them.  Per 64-byte K step a wave loads one
// 16-byte Xq fragment (rows m = lane%16, zero for m >= M) and G 16-byte Wq
// fragments and issues G v_mfma_i32_16x16x64_i8.  The Wq fragments of the
// K steps that hold outlier columns are parked in LDS (with more than 8 such
// steps they are used at once instead), and after the weight stream their
// fp16 term is formed from X_O (X values of the outlier
// columns) and W_O = fp16(fp32(Wq*a_w)/127) built from those int8 bytes
// ("LLM.int8() notes", section 2.3: FP16 outlier term; "PyTorch 2.9 supports
// LLM.int8()", section 3: merged at the end): a step with few outlier
// columns with fmas straight into the accumulator layout, a denser one with
// v_mfma_f32_16x16x32_f16 on 16-column fragments.  The 8 per-wave partials
// are summed in LDS in a fixed order (deterministic) and the epilogue writes
// Y = fp16(fp32(C)*a_x*a_w/127^2 + Y_O).
//
// The small loads of the set-up (scales, mask words or rows of X) are
// requested first at kernel entry, then every wave's first two K steps of
// weight, so the weight stream starts with the kernel and the set-up
// (mask words, outlier-step scan, barriers) runs while it arrives.  For up
// to four rows each workgroup derives the mask (column maxima over the
// rows), a_x and the codes of X by itself (16 KiB per row, read from L2 by
// all but the first workgroups) while those loads are in flight: the whole
// call is one launch, with the codes held in LDS ("PyTorch 2.9 supports
// LLM.int8()", section 2: per-row absmax scale of the activations; "LLM.int8()
// notes", section 3.2: outlier columns are those whose magnitude exceeds the
// threshold).
#include "device_common.h"
#include "launch.h"
#include "tile_layout.h"

namespace i8mm {

namespace {
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kU = 2;  // K steps per loop iteration
constexpr int kSlots = 8;  // outlier K steps parked in LDS (more: static schedule)
constexpr int kSparseCols = 4;  // outlier columns per step taken one by one (fma form)
constexpr int kMaxWords = (133144 + 63) / 64 * 2;  // mask words for the largest K
// single-row calls code X in the kernel up to this padded row length (its
// codes are held in LDS beside the reduction and outlier-slot buffers)
constexpr int kRowMaxLdk = 16384;
// two to four rows coded here: up to this padded row length
constexpr int kRowsMaxLdk = 8192;
// ... and up to this many groups of 16 weight rows per workgroup (LDS)
constexpr int kRowsMaxG = 7;
// padded row length and 8-column chunks per thread and row, by RR
constexpr int row_max_ldk(int rr) { return rr == 1 ? kRowMaxLdk : kRowsMaxLdk; }
constexpr int row_chunks(int rr) { return rr == 0 ? 1 : row_max_ldk(rr) / 8 / kThreads; }
}  // namespace

// A 16-byte Wq fragment.  The weight is read once per call and never again
// in it: nontemporal loads (measured 4.95 -> 5.55 TB/s over the
// 8192 x 28672 weight) keep it from displacing what the caches do reuse.
__device__ __forceinline__ v4i wload(const int8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

// RR > 0: the M <= RR rows of X coded here (Xq, x_scale and mask_bits
// unused; RR = 1 for one row, RR = 4 for two to four rows, which repeat row
// M-1 up to four); RR = 0: the codes, scales and mask words come from the
// activation pass.
template <int G, int MODE, int RR>  // MODE 0: Y, 1: int32 C
__global__ __launch_bounds__(kThreads) void k_gemm_decode(
    const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq, int M, int N, int K, int ldk,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale,
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ mask_bits, float threshold,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C) {
  constexpr bool ROW = RR > 0;
  constexpr int kRC = row_chunks(RR);                     // chunks per thread and row
  constexpr int kXqRow = ROW ? row_max_ldk(RR) / 16 : 1;  // s_xq fragments per row
  __shared__ uint32_t s_bits[ROW ? kRowMaxLdk / 32 : kMaxWords];
  __shared__ int s_red[kWaves][G * 256];
  __shared__ v4i s_wslot[kSlots][G][64];  // Wq fragments of the outlier steps
  __shared__ v4i s_xq[ROW ? RR * kXqRow : 1];  // ROW: the codes of X, row by row
  __shared__ uint32_t s_wmax[ROW ? RR : 1][kWaves];
  __shared__ int s_slot_step[kSlots];
  __shared__ int s_nslots;
  __shared__ int s_next;
  __shared__ float s_aw[G * 16];    // w_scale of the workgroup's rows
  __shared__ uint32_t s_bias[G * 16];  // their biases' binary16 bits (0 without)
  __shared__ float s_ax[16];        // x_scale of the rows (activation pass)

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nw = ldk / 32;
  const int nsteps = ldk / 64;

  const int n_base = blockIdx.x * (G * 16);
  const int ml = lane & 15;   // row of the Xq fragment / column of the result
  const int kq = (lane >> 4) * 16;  // byte offset of this lane inside the 64-byte step

  // panel-tiled operands (tile_layout.h): step s of row r is at
  // tiled_offset(r, 64*s + kq) = tiled_offset(r, kq) + s * 16 KiB; the 16 rows
  // of a group are 1 KiB contiguous per step
  const int8_t* xrow = ROW ? nullptr : Xq + tiled_offset(ml, kq, ldk);
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

  // Loads of the kU steps base .. base+kU-1 (steps past the last re-read the
  // last one; their X fragments are zero, so they add nothing).
  auto load_w = [&](int base, v4i (&b)[kU][G]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t off = (size_t)min(base + u, nsteps - 1) * kTileBytes;
#pragma unroll
      for (int g = 0; g < G; ++g) b[u][g] = wload(wrow[g] + off);
    }
  };
  auto load_x = [&](int base, v4i (&a)[kU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int st = base + u;
      if constexpr (ROW)
        a[u] = (ml < M && st < nsteps) ? s_xq[ml * kXqRow + ((st * 64 + kq) >> 4)] : v4i{};
      else
        a[u] = (xvalid && st < nsteps) ? *reinterpret_cast<const v4i*>(xrow + (size_t)st * kTileBytes)
                                       : v4i{};
    }
  };

  // wave w's first chunk: steps w*kU .. w*kU+kU-1, requested before the
  // set-up.  (With 8 groups per workgroup the extra chunk would not fit the
  // registers: there every step goes through the schedules below.)
  constexpr bool kEarly = G <= 7;
  const int first = kEarly ? wave * kU : ldk;
  // The set-up's own loads go first: loads complete in issue order, so
  // requested after the first weight chunk they would hold the set-up until
  // the whole chunk had arrived (and the next chunk is requested only after
  // the set-up).  The scales and biases the fp16 outlier pass and the
  // epilogue need (one value per thread, into LDS at the set-up's barrier),
  // the first mask words (activation pass) or the rows of X (coded here).
  const int sn = min(n_base + t, N - 1);
  const float pre_aw = t < G * 16 ? w_scale[sn] : 0.0f;
  // (the bias as its bits, converted where it is used: a conversion here
  // would wait for the load at once)
  const uint16_t pre_b = t < G * 16 && bias != nullptr ? bias[sn] : (uint16_t)0;
  const float pre_ax = !ROW && t < 16 && t < M ? x_scale[t] : 0.0f;
  const uint32_t pre_mw = !ROW && t < nw ? mask_bits[t] : 0u;
  const int nck = K >> 3;  // ROW: whole 8-column chunks of the row
  uint4 hv[ROW ? RR * kRC : 1];  // row r's chunk t + u*kThreads at hv[r*kRC + u]
  if constexpr (ROW) {
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const uint4* xr = reinterpret_cast<const uint4*>(X + (size_t)min(r, M - 1) * K);
#pragma unroll
      for (int u = 0; u < kRC; ++u) {
        const int c = t + u * kThreads;
        hv[r * kRC + u] = c < nck ? xr[c] : uint4{0u, 0u, 0u, 0u};
      }
    }
  }
  v4i b[kU][G];
  v4i a[kU];
  if constexpr (kEarly) {
    load_w(first, b);
    if constexpr (!ROW) load_x(first, a);
  }

  if (t == 0) {
    s_nslots = 0;
    s_next = kEarly ? kWaves * kU : 0;  // the dynamic schedule hands out the steps after the first chunks
  }
  float ax = 0.0f;  // ROW: a_x of the row
  // ROW: the row's 8-column chunks that hold outlier columns, kept in the
  // reduction buffer (unused until the end) for the fp16 pass; needs
  // kRowMaxLdk*2 bytes there (G >= 4)
  constexpr bool kRowStash = RR == 1 && G * 256 * kWaves * 4 >= kRowMaxLdk * 2;
  uint4* s_xrow = reinterpret_cast<uint4*>(&s_red[0][0]);
  if constexpr (ROW) {
    // mask bytes (strict colmax > threshold over the rows; padding columns
    // k >= K never), each row's absmax over the regular columns, then the
    // codes of the rows into LDS
    const int nch = ldk / 8;
    uint8_t* s_ob = reinterpret_cast<uint8_t*>(s_bits);  // mask byte of chunk c
    uint32_t ob[kRC];
#pragma unroll
    for (int u = 0; u < kRC; ++u) {
      const int c = t + u * kThreads;
      uint32_t m4[4] = {0u, 0u, 0u, 0u};  // |x| bits, two columns per word
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        const uint4 h = hv[r * kRC + u];
        m4[0] = pk_max_u16(m4[0], h.x & 0x7fff7fffu);
        m4[1] = pk_max_u16(m4[1], h.y & 0x7fff7fffu);
        m4[2] = pk_max_u16(m4[2], h.z & 0x7fff7fffu);
        m4[3] = pk_max_u16(m4[3], h.w & 0x7fff7fffu);
      }
      uint32_t o = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o |= (h2f((uint16_t)((m4[i >> 1] >> ((i & 1) * 16)) & 0xffffu)) > threshold ? 1u : 0u) << i;
      ob[u] = o;
      if (c < nch) s_ob[c] = (uint8_t)o;
    }
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      uint32_t mx2 = 0;
#pragma unroll
      for (int u = 0; u < kRC; ++u) mx2 = pk_max_u16(mx2, chunk_absmax2(hv[r * kRC + u], ob[u]));
      const uint32_t mw = wave_max(max(mx2 & 0xffffu, mx2 >> 16));
      if (lane == 0) s_wmax[r][wave] = mw;
    }
    __syncthreads();
    uint2* s_xq2 = reinterpret_cast<uint2*>(s_xq);
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      uint32_t mx = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = max(mx, s_wmax[r][w]);
      const float axr = h2f((uint16_t)mx);
      if (r == 0) ax = axr;
      if (RR > 1 && t == r && r < M) s_ax[r] = axr;
      const float rr = axr == 0.0f ? 0.0f : 127.0f / axr;
#pragma unroll
      for (int u = 0; u < kRC; ++u) {
        const int c = t + u * kThreads;
        if (r < M && c < nch) {
          const uint4 h = hv[r * kRC + u];
          float dev;
          uint2 q = quant8_fast(h, rr, &dev);
          if (dev > kTieGuard) q = quant8_exact(h, axr);
          q.x &= keep_bytes(ob[u] & 0xfu);
          q.y &= keep_bytes(ob[u] >> 4);
          s_xq2[r * (kXqRow * 2) + c] = q;
          // the X values of the chunk's outlier columns, for the fp16 pass
          if (kRowStash && ob[u] != 0u) s_xrow[c] = h;
        }
      }
    }
  } else {
    if (t < nw) s_bits[t] = pre_mw;
    for (int w = t + kThreads; w < nw; w += kThreads) s_bits[w] = mask_bits[w];
  }
  if (t < G * 16) {
    s_aw[t] = pre_aw;
    s_bias[t] = pre_b;
  }
  if (!ROW && t < 16) s_ax[t] = pre_ax;
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
  // Few outlier steps: the int8 work after the first chunks is handed out
  // dynamically (the waves of a workgroup finish together instead of the
  // slowest setting the pace) and the outlier steps' Wq fragments are parked
  // in LDS for a fixed-order fp16 pass at the end (the result stays
  // deterministic).  Many: static split with the outlier term inline.
  const bool dynamic = n_oslots <= kSlots;

  v4i acc[G];
  v4f acco[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    acc[g] = v4i{};
    acco[g] = v4f{};
  }

  // fp16 outlier term of step s for this lane's 16 columns k0 .. k0+15 (bw:
  // the step's Wq fragments, already in registers)
  auto outlier_step = [&](int s, const v4i (&bw)[G]) __attribute__((always_inline)) {
    const int k0 = s * 64 + kq;
    const uint32_t obits = (s_bits[k0 >> 5] >> (k0 & 31)) & 0xffffu;
    v8h xa[2];
    if constexpr (kRowStash) {
      // the two stashed chunks of columns k0 .. k0+15 (only their outlier
      // entries were written and only those are used)
      const uint4 c0 = s_xrow[k0 >> 3], c1 = s_xrow[(k0 >> 3) + 1];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uint16_t v = 0;
        if (((obits >> e) & 1u) && xvalid) v = (uint16_t)half_at(e < 8 ? c0 : c1, e & 7);
        xa[e >> 3][e & 7] = __builtin_bit_cast(_Float16, v);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uint16_t v = 0;
        if (((obits >> e) & 1u) && xvalid) v = X[(size_t)ml * K + k0 + e];
        xa[e >> 3][e & 7] = __builtin_bit_cast(_Float16, v);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float aw = s_aw[g * 16 + ml];
      v8h wb[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uint16_t v = 0;
        if ((obits >> e) & 1u) {
          const int q = (int)(int8_t)((bw[g][e >> 2] >> ((e & 3) * 8)) & 0xff);
          v = dequant_w_half(q, aw);
        }
        wb[e >> 3][e & 7] = __builtin_bit_cast(_Float16, v);
      }
      acco[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], wb[0], acco[g], 0, 0, 0);
      acco[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], wb[1], acco[g], 0, 0, 0);
    }
  };
  auto step_has_outliers = [&](int s) { return (s_bits[2 * s] | s_bits[2 * s + 1]) != 0u; };

  // MFMAs of a loaded chunk; its outlier steps parked in their LDS slots
  // (dynamic schedule) or accumulated at once (static)
  auto mfma_chunk = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][g], acc[g], 0, 0, 0);
  };
  auto park_chunk = [&](int base) __attribute__((always_inline)) {
    if (!has_outliers) return;
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
  };
  auto inline_chunk = [&](int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int st = min(base + u, nsteps - 1);
      if (base + u < nsteps && step_has_outliers(st)) outlier_step(st, b[u]);
    }
  };

  // The prefetched chunk.  In the static schedule its outlier steps come at
  // the end, their weight fragments read a second time (many outlier steps
  // only: at most kU of them per wave).
  if (kEarly && first < nsteps) {
    if constexpr (ROW) load_x(first, a);
    mfma_chunk();
    if (dynamic) park_chunk(first);
  }
  if (dynamic) {
    // chunks of kU steps from a workgroup counter, fetched one chunk ahead
    int base = 0;
    if (lane == 0) base = atomicAdd(&s_next, kU);
    base = __builtin_amdgcn_readfirstlane(base);
    while (base < nsteps) {
      int nb = 0;
      if (lane == 0) nb = atomicAdd(&s_next, kU);
      load_w(base, b);
      load_x(base, a);
      mfma_chunk();
      park_chunk(base);
      base = __builtin_amdgcn_readfirstlane(nb);
    }
    __syncthreads();
    // fp16 outlier term, slot k on wave k % kWaves, in slot order
    for (int k = wave; k < n_oslots; k += kWaves) {
      const int st = s_slot_step[k];
      // A step with few outlier columns: each column's products x[m] *
      // W_O[n] added with fmas straight into the accumulator (lane l holds
      // rows m = 4 (l / 16) + r, r < 4, of column n = n_base + 16 g + l % 16),
      // the int8 code read from the parked fragment of the lane that loaded
      // it (byte c % 16 of lane l % 16 + 16 (c / 16)) -- the same single
      // rounding per product as the MFMA form, without building 16-column
      // fragments that are almost all zero.  X values: the stashed row (one
      // row), else X itself.
      if (RR != 1 || kRowStash) {
        uint64_t cols = ((uint64_t)s_bits[2 * st + 1] << 32) | s_bits[2 * st];
        if (__popcll(cols) <= kSparseCols) {
          const uint32_t* slot32 = reinterpret_cast<const uint32_t*>(&s_wslot[k][0][0]);
          while (cols != 0ull) {
            const int c = __builtin_ctzll(cols);  // column within the step (wave-uniform)
            cols &= cols - 1ull;
            const int col = st * 64 + c;
            const int src = (lane & 15) + 16 * (c >> 4);
            if constexpr (RR == 1) {
              // the single row is row 0 of the accumulator: lanes 0..15, element 0
              const float x = h2f((uint16_t)half_at(s_xrow[col >> 3], col & 7));
#pragma unroll
              for (int g = 0; g < G; ++g) {
                const uint32_t word = slot32[(g * 64 + src) * 4 + ((c & 15) >> 2)];
                const int q = (int)(int8_t)((word >> ((c & 3) * 8)) & 0xffu);
                const float wo = h2f(dequant_w_half(q, s_aw[g * 16 + (lane & 15)]));
                if (lane < 16) acco[g][0] = fmaf(x, wo, acco[g][0]);
              }
            } else {
              float xr[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int m = 4 * (lane >> 4) + r;
                xr[r] = m < M ? h2f(X[(size_t)m * K + col]) : 0.0f;
              }
#pragma unroll
              for (int g = 0; g < G; ++g) {
                const uint32_t word = slot32[(g * 64 + src) * 4 + ((c & 15) >> 2)];
                const int q = (int)(int8_t)((word >> ((c & 3) * 8)) & 0xffu);
                const float wo = h2f(dequant_w_half(q, s_aw[g * 16 + (lane & 15)]));
#pragma unroll
                for (int r = 0; r < 4; ++r) acco[g][r] = fmaf(xr[r], wo, acco[g][r]);
              }
            }
          }
          continue;
        }
      }
      v4i bw[G];
#pragma unroll
      for (int g = 0; g < G; ++g) bw[g] = s_wslot[k][g][lane];
      outlier_step(st, bw);
    }
  } else {
    // the steps after the first chunks split evenly over the waves, kU per
    // iteration: all their loads are issued before the first MFMA, so a
    // wave keeps kU*G KiB of weight reads in flight
    const int done = kEarly ? min(kWaves * kU, nsteps) : 0;
    const int s0 = done + ((nsteps - done) * wave) / kWaves;
    const int s1 = done + ((nsteps - done) * (wave + 1)) / kWaves;
    int s = s0;
    for (; s + kU <= s1; s += kU) {
      load_w(s, b);
      load_x(s, a);
      mfma_chunk();
      inline_chunk(s);
    }
    for (; s < s1; ++s) {
      const size_t off = (size_t)s * kTileBytes;
      v4i bw[G];
#pragma unroll
      for (int g = 0; g < G; ++g) bw[g] = wload(wrow[g] + off);
      v4i xa1;
      if constexpr (ROW)
        xa1 = ml == 0 ? s_xq[(s * 64 + kq) >> 4] : v4i{};
      else
        xa1 = xvalid ? *reinterpret_cast<const v4i*>(xrow + off) : v4i{};
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa1, bw[g], acc[g], 0, 0, 0);
      if (step_has_outliers(s)) outlier_step(s, bw);
    }
    for (int st = first; st < min(first + kU, nsteps); ++st) {
      if (!step_has_outliers(st)) continue;
      v4i bw[G];
#pragma unroll
      for (int g = 0; g < G; ++g) bw[g] = wload(wrow[g] + (size_t)st * kTileBytes);
      outlier_step(st, bw);
    }
  }

  // the stashed row lives in the reduction buffer: every wave is done with it
  if constexpr (kRowStash) __syncthreads();

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
      const float sc = (RR == 1 ? ax : s_ax[m]) * s_aw[g * 16 + (ln & 15)] * kInv127Sq;
      const float b = h2f((uint16_t)s_bias[g * 16 + (ln & 15)]);
      Y[(size_t)m * N + n] = f2h((float)csum[u] * sc + osum[u] + b);
    }
  }
}

// 16-row weight groups per workgroup: spread over the 256 CUs, 1 .. 8.
static int decode_groups_per_workgroup(int N) {
  const int groups = (N + 15) / 16;
  int G = (groups + 255) / 256;
  if (G > 8) G = 8;
  if (G < 1) G = 1;
  return G;
}

template <int G>
static void launch_g(dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const int8_t* Xq, const int8_t* Wq, int M, int N,
                     int K, int ldk, const float* xs, const float* ws, const uint16_t* X,
                     const uint32_t* mb, float threshold, const uint16_t* bias, uint16_t* Y,
                     int32_t* C) {
  if (Xq == nullptr) {  // the rows of X coded in the kernel
    if (M == 1)
      hipExtLaunchKernelGGL((k_gemm_decode<G, 0, 1>), grid, dim3(kThreads), 0, s, e0, e1, 0, Xq,
                            Wq, M, N, K, ldk, xs, ws, X, mb, threshold, bias, Y, C);
    else if constexpr (G <= kRowsMaxG)  // (gemm_decode_row_ok admits no other)
      hipExtLaunchKernelGGL((k_gemm_decode<G, 0, 4>), grid, dim3(kThreads), 0, s, e0, e1, 0, Xq,
                            Wq, M, N, K, ldk, xs, ws, X, mb, threshold, bias, Y, C);
  } else if (C != nullptr)
    hipExtLaunchKernelGGL((k_gemm_decode<G, 1, 0>), grid, dim3(kThreads), 0, s, e0, e1, 0, Xq,
                          Wq, M, N, K, ldk, xs, ws, X, mb, threshold, bias, Y, C);
  else
    hipExtLaunchKernelGGL((k_gemm_decode<G, 0, 0>), grid, dim3(kThreads), 0, s, e0, e1, 0, Xq,
                          Wq, M, N, K, ldk, xs, ws, X, mb, threshold, bias, Y, C);
}

// Xq == nullptr: the form that codes the rows of X itself (M <= 4, Y output).
static hipError_t launch_decode(const int8_t* Xq, const int8_t* Wq, int M, int N, int K, int ldk,
                                const float* x_scale, const float* w_scale, const uint16_t* X,
                                const uint32_t* mask_bits, float threshold, const uint16_t* bias,
                                uint16_t* Y, int32_t* C, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1) {
  // Spread the 16-row groups evenly over the 256 CUs: G groups per workgroup.
  const int groups = (N + 15) / 16;
  const int G = decode_groups_per_workgroup(N);
  dim3 grid((groups + G - 1) / G);
#define I8MM_DECODE_G(g)                                                                  \
  case g:                                                                                 \
    launch_g<g>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, \
                threshold, bias, Y, C);                                                   \
    break;
  switch (G) {
    I8MM_DECODE_G(1)
    I8MM_DECODE_G(2)
    I8MM_DECODE_G(3)
    I8MM_DECODE_G(4)
    I8MM_DECODE_G(5)
    I8MM_DECODE_G(6)
    I8MM_DECODE_G(7)
    default:
      launch_g<8>(grid, s, e0, e1, Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits,
                  threshold, bias, Y, C);
      break;
  }
#undef I8MM_DECODE_G
  return hipGetLastError();
}

hipError_t launch_gemm_decode(const int8_t* Xq, const int8_t* Wq, int M, int N, int K, int ldk,
                              const float* x_scale, const float* w_scale, const uint16_t* X,
                              const uint32_t* mask_bits, const uint16_t* bias, uint16_t* Y,
                              int32_t* C, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (Xq == nullptr) return hipErrorInvalidValue;
  return launch_decode(Xq, Wq, M, N, K, ldk, x_scale, w_scale, X, mask_bits, 0.0f, bias, Y, C,
                       s, e0, e1);
}

bool gemm_decode_row_ok(const uint16_t* X, int M, int K, int ldk, int N) {
  return M >= 1 && M <= 4 && K > 0 && (K % 8) == 0 &&
         (reinterpret_cast<uintptr_t>(X) & 15) == 0 &&
         ldk <= (M == 1 ? kRowMaxLdk : kRowsMaxLdk) &&
         (M == 1 || decode_groups_per_workgroup(N) <= kRowsMaxG);
}

hipError_t launch_gemm_decode_row(const uint16_t* X, int M, int K, int ldk, float threshold,
                                  const int8_t* Wq, int N, const float* w_scale,
                                  const uint16_t* bias, uint16_t* Y, hipStream_t s, hipEvent_t e0,
                                  hipEvent_t e1) {
  if (!gemm_decode_row_ok(X, M, K, ldk, N) || Y == nullptr) return hipErrorInvalidValue;
  return launch_decode(nullptr, Wq, M, N, K, ldk, nullptr, w_scale, X, nullptr, threshold, bias,
                       Y, nullptr, s, e0, e1);
}

}  // namespace i8mm
