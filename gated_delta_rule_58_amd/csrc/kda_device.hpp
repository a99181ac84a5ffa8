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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays NaN): gfx950
// converts in hardware (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Workgroup barrier for LDS traffic: this wave's LDS operations have completed
// (lgkmcnt 0) before it arrives, while its global loads and stores stay in
// flight (the release fence of __syncthreads would wait for those too, which
// drains any prefetch issued before the barrier).  The empty asm statements
// keep the compiler from moving memory operations across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw element loads: the bits as stored (bf16 kept as uint16), widened to
// fp32 only where used, so that a load stays in flight across the work
// between its issue and its use.
template <bool BF16>
struct Raw {
  typedef float T1;
  typedef f32x4 T4;
};
template <>
struct Raw<true> {
  typedef uint16_t T1;
  typedef u16x4 T4;
};
template <bool BF16>
__device__ __forceinline__ typename Raw<BF16>::T1 load1_raw(const void* base, int64_t idx) {
  return static_cast<const typename Raw<BF16>::T1*>(base)[idx];
}
template <bool BF16>
__device__ __forceinline__ typename Raw<BF16>::T4 load4_raw(const void* base, int64_t idx) {
  return *reinterpret_cast<const typename Raw<BF16>::T4*>(
      static_cast<const typename Raw<BF16>::T1*>(base) + idx);
}
template <bool BF16>
__device__ __forceinline__ float widen1(typename Raw<BF16>::T1 r) {
  if constexpr (BF16) return bf16_bits_to_f32(r);
  else return r;
}
template <bool BF16>
__device__ __forceinline__ f32x4 widen4(typename Raw<BF16>::T4 r) {
  if constexpr (BF16)
    return f32x4{bf16_bits_to_f32(r[0]), bf16_bits_to_f32(r[1]), bf16_bits_to_f32(r[2]),
                 bf16_bits_to_f32(r[3])};
  else return r;
}

// Raw buffer resource over [base, base + nbytes): loads past the end return 0
// and stores past the end are dropped (nbytes = 0 masks every access without
// a branch).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}
constexpr int kBufNT = 2;  // buffer access cache policy: non-temporal

// Holds x in its register until this point: nothing computed from x (a
// widening, say) can be moved above it, so a load of x issued earlier stays
// in flight up to here.
template <typename T>
__device__ __forceinline__ void hold(T& x) {
  asm volatile("" : "+v"(x));
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
