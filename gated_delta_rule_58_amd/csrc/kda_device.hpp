// Device-side helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Load 4 consecutive elements (bf16 or fp32) as fp32.
__device__ __forceinline__ f32x4 load4(const void* base, int64_t idx, bool is_bf16) {
  if (is_bf16) {
    const u16x4 r = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(base) + idx);
    return f32x4{bf16_bits_to_f32(r[0]), bf16_bits_to_f32(r[1]), bf16_bits_to_f32(r[2]),
                 bf16_bits_to_f32(r[3])};
  }
  return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
}

__device__ __forceinline__ float load1(const void* base, int64_t idx, bool is_bf16) {
  if (is_bf16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  return static_cast<const float*>(base)[idx];
}

__device__ __forceinline__ void store4(void* base, int64_t idx, f32x4 v, bool is_bf16) {
  if (is_bf16) {
    u16x4 r = {f32_to_bf16_bits(v[0]), f32_to_bf16_bits(v[1]), f32_to_bf16_bits(v[2]),
               f32_to_bf16_bits(v[3])};
    *reinterpret_cast<u16x4*>(static_cast<uint16_t*>(base) + idx) = r;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = v;
  }
}

}  // namespace kda
