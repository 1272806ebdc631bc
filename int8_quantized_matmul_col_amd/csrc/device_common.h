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

}  // namespace i8mm
