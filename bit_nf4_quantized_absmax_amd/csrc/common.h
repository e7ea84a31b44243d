// Shared device helpers for the gfx950 kernels of libqlora_mi355x.
//
// Everything here is compiled with -ffp-contract=off: the codec steps are
// defined with separate fp32 roundings (a product, then a sum), and a fused
// multiply-add would change their bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_tables.h"

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBlock = 64;    // weights per first-level absmax block
constexpr int kGroup = 256;   // first-level constants per second-level group

__device__ __forceinline__ float u2f(uint32_t b) { return __uint_as_float(b); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even.  Lowers to
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}

// Code of the zero level of each 4-bit table (NF4, FP4, Int4): written for
// every element of a block whose constant is 0.
__device__ __forceinline__ int q4_zero_code(int qtype) { return qtype == 2 ? 8 : 7; }

// Block constant decode: c_hat = fl32(fl32(t8 * c2) + mean), two roundings.
__device__ __forceinline__ float decode_absmax(float t8_level, float c2, float mean) {
  float prod = t8_level * c2;
  return prod + mean;
}

// Wave-wide (64-lane) reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t ceil_div_u32(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

}  // namespace qlora
