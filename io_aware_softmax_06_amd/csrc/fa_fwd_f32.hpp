// Attention forward in float32 end to end (inputs, arithmetic, output).
//
// The same one-pass recurrence as the bf16 kernel (wmrh.cn FlashAttention
// article, section 2.2), on the vector ALU: one wave per workgroup, four lanes
// per query row (each holding a quarter of the d components, the dot products
// completed with two lane exchanges), so 16 rows per workgroup; 32-key tiles
// of K and V staged in LDS and read as broadcasts.  Four lanes per row rather
// than one keep each lane's dependent chain of FMAs short: with one row per
// lane a small launch (B = H = 1, N = 256) ran four single-wave workgroups
// whose serial dot products set its time.
// This is the exact-precision variant; bf16 inputs take the MFMA kernel.
// In kSplit mode the workgroup covers the key range of one split and writes
// the partial result described at ModeArgs (fa_common.hpp) instead of O, L;
// in kSparse mode it skips the 64-key blocks its query block does not see
// (the workgroup's rows lie in one 64-row block of the mask).
#pragma once

#include "fa_common.hpp"

namespace FA355_NS {

// Keys per staged tile: 32, or 16 at d = 256 (two f32 tiles of 16 KB each).
template <int D>
constexpr int kF32Keys = D > 128 ? 16 : 32;
// Lanes per query row and query rows per workgroup (the host sizes its grid
// with kF32Rows).
constexpr int kF32LanesPerRow = 4;
constexpr int kF32Rows = 64 / kF32LanesPerRow;

template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(64) void fa_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ Lse, int N, int BH, int num_qtiles, float scale,
    float scale_log2, ModeArgs split_args) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dimension");
  constexpr int kKeys = kF32Keys<D>;
  constexpr bool SPLIT = MODE == kSplit;
  constexpr bool SPARSE = MODE == kSparse;
  constexpr int kLanesPerRow = kF32LanesPerRow;
  constexpr int kRows = kF32Rows;           // query rows per workgroup
  constexpr int kDl = D / kLanesPerRow;     // components of d held per lane
  static_assert(kDl % 4 == 0, "whole float4 pieces per lane");
  __shared__ f32x4 ks[kKeys][D / 4];
  __shared__ f32x4 vs[kKeys][D / 4];

  const int lane = threadIdx.x;
  const int part = lane / kRows;  // which quarter of the d components
  int split = 0, wg = blockIdx.x;
  if (SPLIT) {
    split = wg % split_args.num_splits;
    wg /= split_args.num_splits;
  }
  const int bh = wg / num_qtiles;
  int qt = wg - bh * num_qtiles;
  if (CAUSAL) qt = num_qtiles - 1 - qt;
  const int q0 = qt * kRows;
  const int qrow = q0 + lane % kRows;
  const size_t head = (size_t)bh * N * D;

  f32x4 q[kDl / 4], o[kDl / 4];
#pragma unroll
  for (int t = 0; t < kDl / 4; ++t) {
    q[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (qrow < N)
      q[t] = *reinterpret_cast<const f32x4*>(Q + head + (size_t)qrow * D + part * kDl + 4 * t);
  }
  // m_run: largest raw score so far; base_run = fl(m_run * scale_log2), the
  // base-2 reference of l_run and o (-inf until a visible key is seen), kept
  // rounded so that exp2(base_old - base_new) rescales exactly.
  float m_run = kNegInf, base_run = kNegInf, l_run = 0.f;

  // Keys of this workgroup: [kv_lo, kv_hi), the range of its split for its
  // 256-row block (kRows divides 256, so the workgroup lies in one block).
  static_assert(kSplitRows % kRows == 0, "row blocks");
  int kv_lo = 0, kv_hi = N;
  if (SPLIT) split_range(split, split_args.num_splits, q0 / kSplitRows, N, CAUSAL, kv_lo, kv_hi);
  const int kv_end = CAUSAL ? min(kv_hi, q0 + kRows) : kv_hi;
  static_assert(kMaskBlock % kKeys == 0 && kMaskBlock % kRows == 0, "mask blocks");
  const int nb = (N + kMaskBlock - 1) / kMaskBlock;
  const uint8_t* mrow = nullptr;
  if (SPARSE)
    mrow = split_args.mask +
           ((size_t)mask_head(split_args, bh) * nb + q0 / kMaskBlock) * (size_t)nb;
  for (int kv0 = kv_lo; kv0 < kv_end; kv0 += kKeys) {
    if (SPARSE && mrow[kv0 / kMaskBlock] == 0) continue;  // same for the whole workgroup
    __syncthreads();
    for (int c = lane; c < kKeys * (D / 4); c += 64) {
      const int row = c / (D / 4), col = c % (D / 4);
      const int key = kv0 + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < kv_end) {
        kv = *reinterpret_cast<const f32x4*>(K + head + (size_t)key * D + 4 * col);
        vv = *reinterpret_cast<const f32x4*>(V + head + (size_t)key * D + 4 * col);
      }
      ks[row][col] = kv;
      vs[row][col] = vv;
    }
    __syncthreads();

    float s[kKeys];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < kDl / 4; ++t) {
        const f32x4 kk = ks[j][part * (kDl / 4) + t];
        acc = __builtin_fmaf(q[t][0], kk[0], acc);
        acc = __builtin_fmaf(q[t][1], kk[1], acc);
        acc = __builtin_fmaf(q[t][2], kk[2], acc);
        acc = __builtin_fmaf(q[t][3], kk[3], acc);
      }
      if (kLanesPerRow >= 2) acc += other_half(acc);
      if (kLanesPerRow == 4) acc += __shfl_xor(acc, 16, 64);
      const int key = kv0 + j;
      s[j] = (key >= kv_end || (CAUSAL && key > qrow)) ? kNegInf : acc;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float base = (m_new == kNegInf) ? 0.f : m_new * scale_log2;
    const float alpha = fast_exp2(base_run - base);
    base_run = (m_new == kNegInf) ? kNegInf : base;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < kDl / 4; ++t) o[t] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = fast_exp2(__builtin_fmaf(s[j], scale_log2, -base));
      l_run += p;
#pragma unroll
      for (int t = 0; t < kDl / 4; ++t) {
        const f32x4 vv = vs[j][part * (kDl / 4) + t];
        o[t][0] = __builtin_fmaf(p, vv[0], o[t][0]);
        o[t][1] = __builtin_fmaf(p, vv[1], o[t][1]);
        o[t][2] = __builtin_fmaf(p, vv[2], o[t][2]);
        o[t][3] = __builtin_fmaf(p, vv[3], o[t][3]);
      }
    }
    m_run = m_new;
  }

  if (qrow < N) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float r = __builtin_fmaf(m_run, scale_log2, -base_run);  // exact residual
    const float lse = l_run > 0.f ? __builtin_fmaf(m_run, scale, logf(l_run) - r * kLn2) : kNegInf;
    float* orow;
    float* lrow;
    if (SPLIT) {
      const size_t prow = ((size_t)split * BH + bh) * N + qrow;
      orow = split_args.opart + prow * D;
      lrow = split_args.lpart + prow;
    } else {
      orow = O + head + (size_t)qrow * D;
      lrow = Lse + (size_t)bh * N + qrow;
    }
#pragma unroll
    for (int t = 0; t < kDl / 4; ++t)
      *reinterpret_cast<f32x4*>(orow + part * kDl + 4 * t) = o[t] * inv;
    if (part == 0) *lrow = lse;
  }
}

}  // namespace FA355_NS
