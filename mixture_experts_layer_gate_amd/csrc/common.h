// Device-side helpers shared by the kernels of the MoE-layer library (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 storage: the upper 16 bits of an fp32

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element traits: storage type and its conversion to/from fp32.
template <int kDtype> struct Elt;
template <> struct Elt<0> {  // fp32
  typedef float T;
  static constexpr int kBytes = 4;
};
template <> struct Elt<1> {  // bf16
  typedef bf16_t T;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  // SiLU(g) * u = g / (1 + exp(-g)) * u
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace moe
