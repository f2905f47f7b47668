// Attention backward in float32 end to end, on the vector ALU (the
// exact-precision variant; bf16 inputs take the MFMA kernels of
// fa_bwd_bf16.hpp).  Same recomputation and the same two-kernel split as the
// bf16 path: dK and dV stream query tiles past a block of keys, dQ streams
// key tiles past a block of queries.  One wave per workgroup, one row per lane
// (two lanes per row when d = 128, each holding 64 of the d components);
// 32-row tiles of the streamed operands are staged in LDS and read as
// broadcasts.
#pragma once

#include "fa_common.hpp"

namespace FA355_NS {

constexpr int kBwdF32Rows = 32;  // streamed rows per staged tile

// Components of d per lane: all of a row when d <= 64, else 64 (two lanes per
// row at d = 128).
template <int D>
constexpr int kBwdDl = D >= 64 ? 64 : D;

template <int D>
__device__ __forceinline__ float dot_row(const f32x4 (&a)[kBwdDl<D> / 4], const f32x4* b, int part) {
  constexpr int kT = kBwdDl<D> / 4;
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    const f32x4 x = b[part * kT + t];
    acc = __builtin_fmaf(a[t][0], x[0], acc);
    acc = __builtin_fmaf(a[t][1], x[1], acc);
    acc = __builtin_fmaf(a[t][2], x[2], acc);
    acc = __builtin_fmaf(a[t][3], x[3], acc);
  }
  if (D == 128) acc += other_half(acc);
  return acc;
}

// dK, dV: a workgroup owns kRows keys (64 / lanes per row).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fa_bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ Dv,
    float* __restrict__ dK, float* __restrict__ dV, int N, int num_ktiles, float scale,
    float scale_log2) {
  static_assert(D == 32 || D == 64 || D == 128, "head dimension");
  constexpr int kRows = D >= 64 ? 64 / (D / 64) : 64;
  constexpr int kT = kBwdDl<D> / 4;  // f32x4 pieces of d per lane
  __shared__ f32x4 qs[kBwdF32Rows][D / 4];
  __shared__ f32x4 ds_[kBwdF32Rows][D / 4];
  __shared__ float ls[kBwdF32Rows], dls[kBwdF32Rows];

  const int lane = threadIdx.x;
  const int part = lane / kRows;
  const int bh = blockIdx.x / num_ktiles;
  const int k0 = (blockIdx.x - bh * num_ktiles) * kRows;
  const int key = k0 + lane % kRows;
  const size_t head = (size_t)bh * N * D;

  f32x4 k[kT], v[kT], dk[kT], dv[kT];
  const int kr = min(key, N - 1);
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    k[t] = *reinterpret_cast<const f32x4*>(K + head + (size_t)kr * D + part * kBwdDl<D> + 4 * t);
    v[t] = *reinterpret_cast<const f32x4*>(V + head + (size_t)kr * D + part * kBwdDl<D> + 4 * t);
    dk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int q_begin = CAUSAL ? (k0 / kBwdF32Rows) * kBwdF32Rows : 0;
  for (int q0 = q_begin; q0 < N; q0 += kBwdF32Rows) {
    __syncthreads();
    for (int c = lane; c < kBwdF32Rows * (D / 4); c += 64) {
      const int row = c / (D / 4), col = c % (D / 4);
      const int q = q0 + row;
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      if (q < N) {
        a = *reinterpret_cast<const f32x4*>(Q + head + (size_t)q * D + 4 * col);
        b = *reinterpret_cast<const f32x4*>(dO + head + (size_t)q * D + 4 * col);
      }
      qs[row][col] = a;
      ds_[row][col] = b;
    }
    if (lane < kBwdF32Rows) {
      const int q = q0 + lane;
      ls[lane] = q < N ? Lse[(size_t)bh * N + q] : kNegInf;
      dls[lane] = q < N ? Dv[(size_t)bh * N + q] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < kBwdF32Rows; ++i) {
      const int q = q0 + i;
      const float s = dot_row<D>(k, qs[i], part);
      const float nl = ls[i] == kNegInf ? kNegInf : -ls[i] * kLog2e;
      float p = fast_exp2(__builtin_fmaf(s, scale_log2, nl));
      if (q >= N || (CAUSAL && key > q)) p = 0.f;
      const float dp = dot_row<D>(v, ds_[i], part);
      const float dsv = p * (dp - dls[i]);
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        dv[t] += p * ds_[i][part * kT + t];
        dk[t] += dsv * qs[i][part * kT + t];
      }
    }
  }
  if (key < N) {
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      *reinterpret_cast<f32x4*>(dK + head + (size_t)key * D + part * kBwdDl<D> + 4 * t) = dk[t] * scale;
      *reinterpret_cast<f32x4*>(dV + head + (size_t)key * D + part * kBwdDl<D> + 4 * t) = dv[t];
    }
  }
}

// dQ: a workgroup owns kRows queries.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fa_bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ Dv,
    float* __restrict__ dQ, int N, int num_qtiles, float scale, float scale_log2) {
  static_assert(D == 32 || D == 64 || D == 128, "head dimension");
  constexpr int kRows = D >= 64 ? 64 / (D / 64) : 64;
  constexpr int kT = kBwdDl<D> / 4;  // f32x4 pieces of d per lane
  __shared__ f32x4 ks[kBwdF32Rows][D / 4];
  __shared__ f32x4 vs[kBwdF32Rows][D / 4];

  const int lane = threadIdx.x;
  const int part = lane / kRows;
  const int bh = blockIdx.x / num_qtiles;
  int qt = blockIdx.x - bh * num_qtiles;
  if (CAUSAL) qt = num_qtiles - 1 - qt;
  const int q0 = qt * kRows;
  const int qrow = q0 + lane % kRows;
  const size_t head = (size_t)bh * N * D;

  f32x4 q[kT], g[kT], dq[kT];
  const int qr = min(qrow, N - 1);
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    q[t] = *reinterpret_cast<const f32x4*>(Q + head + (size_t)qr * D + part * kBwdDl<D> + 4 * t);
    g[t] = *reinterpret_cast<const f32x4*>(dO + head + (size_t)qr * D + part * kBwdDl<D> + 4 * t);
    dq[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float lq = Lse[(size_t)bh * N + qr];
  const float nl = lq == kNegInf ? kNegInf : -lq * kLog2e;
  const float drow = Dv[(size_t)bh * N + qr];

  const int kv_end = CAUSAL ? min(N, q0 + kRows) : N;
  for (int kv0 = 0; kv0 < kv_end; kv0 += kBwdF32Rows) {
    __syncthreads();
    for (int c = lane; c < kBwdF32Rows * (D / 4); c += 64) {
      const int row = c / (D / 4), col = c % (D / 4);
      const int kk = kv0 + row;
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
      if (kk < kv_end) {
        a = *reinterpret_cast<const f32x4*>(K + head + (size_t)kk * D + 4 * col);
        b = *reinterpret_cast<const f32x4*>(V + head + (size_t)kk * D + 4 * col);
      }
      ks[row][col] = a;
      vs[row][col] = b;
    }
    __syncthreads();
    for (int j = 0; j < kBwdF32Rows; ++j) {
      const int kk = kv0 + j;
      const float s = dot_row<D>(q, ks[j], part);
      float p = fast_exp2(__builtin_fmaf(s, scale_log2, nl));
      if (kk >= kv_end || (CAUSAL && kk > qrow)) p = 0.f;
      const float dp = dot_row<D>(g, vs[j], part);
      const float dsv = p * (dp - drow);
#pragma unroll
      for (int t = 0; t < kT; ++t) dq[t] += dsv * ks[j][part * kT + t];
    }
  }
  if (qrow < N) {
#pragma unroll
    for (int t = 0; t < kT; ++t)
      *reinterpret_cast<f32x4*>(dQ + head + (size_t)qrow * D + part * kBwdDl<D> + 4 * t) = dq[t] * scale;
  }
}

}  // namespace FA355_NS
