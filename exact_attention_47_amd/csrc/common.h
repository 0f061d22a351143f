// Shared device helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v8f __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef _Float16 v8f16 __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
typedef _Float16 v4f16 __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef _Float16 v2f16 __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr float kNegInf = -__builtin_inff();

// Exchange a value with the lane 32 positions away (the other half of the
// wave) and return the pair's maximum / sum. v_permlane32_swap moves the
// upper half of one operand into the lower half of the other; with the same
// value in both operands each lane sees its own value and its partner's.
__device__ __forceinline__ float pair_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Map a launch-order block id onto a work id so that consecutive work ids
// run on the same XCD: the hardware hands blocks to the 8 XCDs round-robin,
// so block b runs on XCD b % 8. Work ids [x*n/8, (x+1)*n/8) go to XCD x.
// Only used when n is a multiple of 8 (otherwise identity).
__device__ __forceinline__ int xcd_swizzle(int bid, int n) {
  if ((n & 7) != 0) return bid;
  return (bid & 7) * (n >> 3) + (bid >> 3);
}

}  // namespace attn
