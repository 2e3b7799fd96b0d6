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
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kEps = 1e-6f;

// bf16 is the upper half of an fp32: widening is a shift or a mask.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even pack of two floats into bf16x2 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// The low 16-bit halves of a and b as one word (a's in the low half), and
// the high halves likewise: one v_perm_b32 each.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Round-to-nearest-even pack of two floats into fp16x2, and its widenings.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  f16x2_t r = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float h_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[0];
}
__device__ __forceinline__ float h_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[1];
}

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
// The same with the non-temporal hint, for rows read once.
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}
// Store with the non-temporal hint: for results nothing in the same kernel
// reads back, so they leave the cache promptly instead of being written back
// when the kernel ends.
__device__ __forceinline__ void st16_nt(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
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

// DPP lane moves within a row of 16 lanes (row_mask/bank_mask all lanes).
template <int ctrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl,
                                                               0xF, 0xF, false));
}

// Sum over groups of `width` consecutive lanes, width in {1, 2, 4, 8, 16},
// with DPP moves only: quad_perm swaps within quads, then half-row and row
// mirrors, which pair every lane with one of the other half once the halves
// below it hold uniform sums.
template <int width>
__device__ __forceinline__ float dpp_group_sum(float x) {
  static_assert(width == 1 || width == 2 || width == 4 || width == 8 || width == 16, "width");
  if constexpr (width >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (width >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (width >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (width >= 16) x += dpp_mov<0x140>(x); // row_mirror
  return x;
}

// x[lane] + x[lane ^ 32].
__device__ __forceinline__ float sum_halves(float x) { return x + __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// Materialise a value in a VGPR at this point of the program (an empty asm
// statement that reads and writes it), so that its computation cannot be
// sunk towards a later use and stays where it was placed in the schedule.
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// dot of two bf16 pairs plus an fp32 addend (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Raw buffer loads: offsets are bytes from the resource base; a load whose
// VGPR offset is at or beyond num_records reads zero (used for ragged tails
// instead of branches). The SGPR offset is not part of that range check, so
// callers move tile offsets into the resource base, never into soffset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_records,
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// The same with the non-temporal hint (cache policy bit 1), for data read
// once: it does not push reused lines out of the caches.
__device__ __forceinline__ u32x4_t bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}
__device__ __forceinline__ u32x2_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

// 16 bytes per lane from a buffer resource straight into LDS, lane i at
// lds + 16*i (buffer_load_dwordx4 ... lds; counted by vmcnt, not lgkmcnt).
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T ceil_div(T a, T b) { return (a + b - 1) / b; }

}  // namespace nc
