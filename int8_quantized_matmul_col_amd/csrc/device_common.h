// Device-side helpers shared by the gfx950 kernels of the decomposed int8
// matmul: vector types for the MFMA operands, float16 bit conversions and the
// absmax quantizer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kQMax = 127;
constexpr float kInv127Sq = 1.0f / 16129.0f;

__device__ __forceinline__ float h2f(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ __forceinline__ uint16_t f2h(float f) {
  // float -> binary16 with round-to-nearest-even (the hardware default mode)
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two floats -> two binary16 (round to nearest even), packed low | high<<16:
// one v_cvt_pk_f16_f32 on gfx950.
__device__ __forceinline__ uint32_t f2h2(float lo, float hi) {
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t{lo, hi}), v2h_t));
}

// |x| of a finite binary16 value, as its bit pattern: for non-negative
// finite values the bit patterns order like the values.
__device__ __forceinline__ uint32_t habs_bits(uint32_t bits) { return bits & 0x7fffu; }

// Absmax quantization code of x against scale a: clamp(rne(fp32(127*x)/a),
// -127, 127), and 0 when a == 0.  127*x is exact in fp32 for binary16 x; the
// division is the IEEE-correctly-rounded fp32 division (the library is built
// without fast-math) and rintf rounds half to even.  For binary16 x and a this
// equals round-half-even of the exact rational 127*x/a.
// Branch-free (selects, no divergent control flow around the division).
__device__ __forceinline__ int quant_code(float x, float a) {
  const bool zero = (a == 0.0f);
  const float d = zero ? 1.0f : a;
  float q = rintf((127.0f * x) / d);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return zero ? 0 : (int)q;
}

// Dequantized outlier weight value fp16(fp32(fp32(q) * a_w) / 127).
__device__ __forceinline__ uint16_t dequant_w_half(int q, float aw) {
  return f2h(((float)q * aw) / 127.0f);
}

__device__ __forceinline__ int pack4_i8(int a, int b, int c, int d) {
  return (a & 0xff) | ((b & 0xff) << 8) | ((c & 0xff) << 16) | ((int)((unsigned)d << 24));
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace i8mm

namespace i8mm {

// Loads the 8 binary16 values row[c0 .. c0+7] (c0 a multiple of 8) into h[],
// with zeros past the row length K.  `vec` says the row start is 16-byte
// aligned and K % 8 == 0, so a full chunk is one 16-byte load.
__device__ __forceinline__ void load8_half(const uint16_t* __restrict__ row, int c0, int K,
                                           bool vec, uint16_t h[8]) {
  if (vec && c0 + 8 <= K) {
    uint4 v = *reinterpret_cast<const uint4*>(row + c0);
    h[0] = v.x & 0xffff; h[1] = v.x >> 16; h[2] = v.y & 0xffff; h[3] = v.y >> 16;
    h[4] = v.z & 0xffff; h[5] = v.z >> 16; h[6] = v.w & 0xffff; h[7] = v.w >> 16;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (c0 + i < K) ? row[c0 + i] : (uint16_t)0;
  }
}

// |v - rint(v)| above this sends a lane to the IEEE division (quant8).
constexpr float kTieGuard = 0.5f - 0x1p-14f;

// binary16 bits of column i (0..7) of a 16-byte chunk.
__device__ __forceinline__ uint32_t half_at(const uint4& w, int i) {
  const uint32_t d = i < 2 ? w.x : i < 4 ? w.y : i < 6 ? w.z : w.w;
  return (i & 1) ? (d >> 16) : (d & 0xffffu);
}

// 16-byte chunk of 8 binary16 values at row[c0], zero past K.
__device__ __forceinline__ uint4 load_chunk(const uint16_t* __restrict__ row, int c0, int K,
                                            bool vec) {
  if (vec && c0 + 8 <= K) return *reinterpret_cast<const uint4*>(row + c0);
  uint32_t d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t lo = (c0 + 2 * p < K) ? row[c0 + 2 * p] : 0u;
    const uint32_t hi = (c0 + 2 * p + 1 < K) ? row[c0 + 2 * p + 1] : 0u;
    d[p] = lo | (hi << 16);
  }
  return uint4{d[0], d[1], d[2], d[3]};
}

__device__ __forceinline__ uint2 pack8_i8(const int (&q)[8]) {
  const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)q[1], (uint32_t)q[0], 0x0c0c0400u);
  const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)q[3], (uint32_t)q[2], 0x0c0c0400u);
  const uint32_t p45 = __builtin_amdgcn_perm((uint32_t)q[5], (uint32_t)q[4], 0x0c0c0400u);
  const uint32_t p67 = __builtin_amdgcn_perm((uint32_t)q[7], (uint32_t)q[6], 0x0c0c0400u);
  return uint2{__builtin_amdgcn_perm(p23, p01, 0x05040100u),
               __builtin_amdgcn_perm(p67, p45, 0x05040100u)};
}

// Codes of the 8 columns of a chunk against the row scale a, with
// r = RN(127/a) (0 when a == 0).  For |x| <= a the exact product x*r lies
// within 2^-17 of the exact 127x/a.  One fma adds 1.5*2^23 to it: the fp32
// sum has unit spacing, so it holds t = the exact product rounded half-even
// to an integer, and its low byte is t's two's-complement code (|t| <= 127;
// no conversion instruction).  t is the exact round-half-even code wherever
// |x*r - t| (one fma) is at most 1/2 - 2^-14; there it also equals rint of
// the IEEE quotient fp32(127x)/a (checked on every binary16 pair
// 0 <= x <= a on the host).  Returns the largest such deviation in *dev:
// above kTieGuard (about 1.5e-4 of the values) the caller recomputes the
// chunk with quant8_exact.  Outlier columns (|x| > a) get arbitrary codes
// here; the caller zeroes them.  Branch-free, so the chunks of a row
// interleave.
__device__ __forceinline__ uint2 quant8_fast(const uint4& w, float r, float* dev) {
  constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
  int q[8];
  float d = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = h2f((uint16_t)half_at(w, i));
    // fma reading the binary16 operand directly; exact integer t after the
    // subtraction (|x*r| < 2^22 on the regular columns)
    const float s = __builtin_fmaf(x, r, kRound);
    const float t = s - kRound;
    d = fmaxf(d, fabsf(__builtin_fmaf(x, r, -t)));
    q[i] = (int)__float_as_uint(s);  // low byte: the code
  }
  *dev = d;
  return pack8_i8(q);
}

// The same codes through the IEEE division (quant_code).
__device__ __forceinline__ uint2 quant8_exact(const uint4& w, float a) {
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = quant_code(h2f((uint16_t)half_at(w, i)), a);
  return pack8_i8(q);
}

// Two-lane unsigned 16-bit max of packed words (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
  const v2u16 m = __builtin_elementwise_max(__builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b));
  return __builtin_bit_cast(uint32_t, m);
}

// Bytes (or binary16 halves) of a chunk that belong to regular columns: the
// mask bits ob (bit i = column i is an outlier) expanded to keep-masks.
__device__ __forceinline__ uint32_t keep_bytes(uint32_t ob4) {
  // bit i of ob4 (< 16) moved to bit 8i (the shifted copies do not overlap),
  // then a byte permute turns each byte into 0x00 (bit set: selector 12) or
  // 0xff (bit clear: selector 13); no full-width multiply
  const uint32_t lsb = (ob4 * 0x00204081u) & 0x01010101u;
  return __builtin_amdgcn_perm(0u, 0u, 0x0d0d0d0du - lsb);
}
// Clear-masks of the outlier columns of one 8-column chunk (mask bits ob,
// bit i = column i), branch-free: v_perm's selectors 8 and 9 fill a byte
// with bit 15 or bit 31 of its second source (10 and 11: of its first), so
// with mask bits moved to bits 15 and 31 of shifted copies of ob, one permute
// makes one mask word.  s3 holds bits 6 and 7 there, s2 bits 4 and 5, s1
// bits 2 and 3, s0 bits 0 and 1 (no other bit of ob reaches 15 or 31).
struct ChunkMasks {
  uint32_t h[4];  // binary16 pair p: 0xffff over column 2p and/or 2p+1 if outliers
  uint32_t b[2];  // code bytes 0-3 and 4-7: 0xff over each outlier column
};
__device__ __forceinline__ ChunkMasks chunk_masks(uint32_t ob) {
  const uint32_t s3 = (ob << 9) | (ob << 24);
  const uint32_t s2 = s3 << 2, s1 = s3 << 4, s0 = s3 << 6;
  ChunkMasks m;
  m.h[0] = __builtin_amdgcn_perm(0u, s0, 0x09090808u);
  m.h[1] = __builtin_amdgcn_perm(0u, s1, 0x09090808u);
  m.h[2] = __builtin_amdgcn_perm(0u, s2, 0x09090808u);
  m.h[3] = __builtin_amdgcn_perm(0u, s3, 0x09090808u);
  m.b[0] = __builtin_amdgcn_perm(s1, s0, 0x0b0a0908u);
  m.b[1] = __builtin_amdgcn_perm(s3, s2, 0x0b0a0908u);
  return m;
}

// Packed |x| maxima (two 16-bit lanes) of the regular columns of a chunk.
__device__ __forceinline__ uint32_t chunk_absmax2(const uint4& w, const ChunkMasks& m) {
  const uint32_t d0 = w.x & ~m.h[0] & 0x7fff7fffu, d1 = w.y & ~m.h[1] & 0x7fff7fffu;
  const uint32_t d2 = w.z & ~m.h[2] & 0x7fff7fffu, d3 = w.w & ~m.h[3] & 0x7fff7fffu;
  return pk_max_u16(pk_max_u16(d0, d1), pk_max_u16(d2, d3));
}
__device__ __forceinline__ uint32_t chunk_absmax2(const uint4& w, uint32_t ob) {
  return chunk_absmax2(w, chunk_masks(ob));
}

}  // namespace i8mm
