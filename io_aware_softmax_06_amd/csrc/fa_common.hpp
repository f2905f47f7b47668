// Shared device helpers for the attention forward kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// each with a private L2.  Renumber so that every XCD receives a contiguous
// run of logical ids: the query tiles of one (batch, head) then run on the
// same XCD and its L2 serves their repeated reads of that head's K and V.
// A bijection on [0, total); ids past the last full round keep their value.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcds = 8;
  const int per = total / kXcds;
  if (bid >= per * kXcds) return bid;
  return (bid % kXcds) * per + bid / kXcds;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// Value held by lane (l ^ 32), the same MFMA column in the other half-wave.
__device__ __forceinline__ float other_half(float v) {
  return __shfl_xor(v, 32, 64);
}

}  // namespace fa355
