// Device helpers shared by the gfx950 kernels: vector types, bf16 <-> f32
// conversion, 16-byte global/LDS access and small wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEps = 1e-6f;

// bf16 is the upper half of an fp32: widening is a shift or a mask.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even pack of two floats into bf16x2 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}
__device__ __forceinline__ void st8(void* p, u32x2_t v) {
  *reinterpret_cast<u32x2_t*>(p) = v;
}

// v_exp_f32: 2^x without the denormal fix-up of exp2f (arguments here are
// bounded well inside the normal range).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = width / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename T>
__device__ __forceinline__ T ceil_div(T a, T b) { return (a + b - 1) / b; }

}  // namespace nc
