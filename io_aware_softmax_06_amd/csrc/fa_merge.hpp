// Merge of key-range partial results into the attention output.
//
// The rule is the softmax of a concatenation from the Triton article's
// section on tiled attention (m = max(m1, m2), l = e^{m1-m} l1 + e^{m2-m} l2),
// extended to the output because the product with V is linear: with each
// range's output O_s already normalised by its own denominator and L_s its
// logsumexp,
//     L = ln sum_s e^{L_s},    O = sum_s e^{L_s - L} O_s.
// A range with no visible key has L_s = -inf and weight 0.
//
// Memory-bound: one thread per 4 consecutive d of a row reads the S partial
// logsumexps of the row (a broadcast within the row's threads) and S float4
// pieces of O_s, and writes 4 outputs; the partials are streamed once.  The
// loops over S are unrolled by 4 so that several independent loads are in
// flight per thread.
#pragma once

#include "fa_common.hpp"

namespace FA355_NS {

constexpr int kMergeThreads = 256;

template <typename OutT>
__device__ __forceinline__ void store4(OutT* p, f32x4 v);

template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, f32x4 v) {
  __bf16 b[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, b);
}

template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* p, f32x4 v) {
  _Float16 b[4] = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, b);
}

// opart [S][rows][D], lpart [S][rows] (rows = B*H*N), O [rows][D], L [rows].
// Grid-stride over rows, so any grid size covers any row count.
template <int D, typename OutT>
__global__ __launch_bounds__(kMergeThreads) void fa_merge_kernel(
    const float* __restrict__ opart, const float* __restrict__ lpart, OutT* __restrict__ O,
    float* __restrict__ L, int S, int64_t rows) {
  constexpr int kPerRow = D / 4;                     // threads per row
  constexpr int kRowsPerBlock = kMergeThreads / kPerRow;
  const int c = threadIdx.x % kPerRow;
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kPerRow; row < rows;
       row += stride) {
    float m = kNegInf;
#pragma unroll 4
    for (int s = 0; s < S; ++s) m = fmaxf(m, lpart[(int64_t)s * rows + row]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != kNegInf) {
#pragma unroll 4
      for (int s = 0; s < S; ++s) {
        // An empty range has ls = -inf, weight exp2(-inf) = 0 and O_s = 0.
        const float ls = lpart[(int64_t)s * rows + row];
        const f32x4 o =
            *reinterpret_cast<const f32x4*>(opart + ((int64_t)s * rows + row) * D + 4 * c);
        const float w = fast_exp2((ls - m) * kLog2e);
        acc += w * o;
        wsum += w;
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    store4<OutT>(O + row * D + 4 * c, acc * inv);
    if (c == 0) L[row] = wsum > 0.f ? m + logf(wsum) : kNegInf;
  }
}

}  // namespace FA355_NS
