// Attention forward, bf16 in / bf16 out, fp32 accumulation, on gfx950 MFMA.
//
// Method: the one-pass tiled attention of the wmrh.cn FlashAttention article
// (section 2.2): one workgroup fixes a block of 128 query rows and streams
// every 64-key block of K and V through LDS, keeping per row the running
// score maximum m, the denominator l relative to m, and the un-normalised
// output.  After the last block the output is divided by l once (the
// rescale-by-e^{m_old - m_new} rule of the Triton article's section on
// tiled attention, applied to l and to the output alike).
//
// gfx950 layout choices:
//  * Each of the 4 waves owns 32 query rows.  Scores are produced transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the accumulator then keeps one
//    query per lane column, so a row's maximum and sum are reduced inside the
//    lane plus one exchange between the two half-waves, and m and l are one
//    scalar per lane.
//  * The output is accumulated transposed too, O^T += V^T P^T: the probability
//    tile P^T goes from the score accumulator into the MFMA B operand without
//    leaving registers.  For that the 32 A-operand rows of the score MFMA are
//    mapped to keys by the permutation `key_of_row` below, chosen so that each
//    half-wave ends up holding 8 consecutive keys per 16-key step.
//  * K is staged row-major in LDS (16-byte reads of 8 consecutive d), V is
//    staged transposed ([d][key]) so that the P V operand is also a 16-byte
//    read of 8 consecutive keys.  Rows are padded by 16 bytes against bank
//    conflicts.
//  * Scores are scaled by scale*log2(e) inside one FMA and exponentiated with
//    v_exp_f32 (base 2); L is formed in natural-log units at the end.
#pragma once

#include "fa_common.hpp"

namespace fa355 {

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kThreads = 256;  // 4 waves x 32 query rows

template <int D>
struct Bf16Smem {
  static constexpr int kStride = D + 8;    // bf16 per staged K row
  static constexpr int vStride = kBN + 8;  // bf16 per staged V^T row
  uint16_t ks[kBN * kStride];
  uint16_t vt[D * vStride];
};

// Key (within a 32-key block) fed to A-operand row i of the score MFMA.  With
// i = 8g + 4h + r (g = 0..3, h = 0..1, r = 0..3) the accumulator element
// 4g + r of half-wave h holds row i; this mapping makes the elements
// 8s .. 8s+7 of half-wave h equal the keys 16s + 8h + (0..7), s = 0..1.
__device__ __forceinline__ int key_of_row(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + r;
}

__device__ __forceinline__ bf16x8 lds_read_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

template <int D>
__device__ __forceinline__ void stage_kv_tile(Bf16Smem<D>& sm, const uint16_t* __restrict__ Kb,
                                              const uint16_t* __restrict__ Vb, int kv0, int N,
                                              int tid) {
  constexpr int kChunksPerRow = D / 8;  // 16-byte chunks in a row of K or V
  // K: row-major copy, consecutive threads take consecutive 16-byte chunks.
#pragma unroll
  for (int c = tid; c < kBN * kChunksPerRow; c += kThreads) {
    const int row = c / kChunksPerRow;
    const int col = (c % kChunksPerRow) * 8;
    const int key = kv0 + row;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < N) val = *reinterpret_cast<const u32x4*>(Kb + (size_t)key * D + col);
    *reinterpret_cast<u32x4*>(&sm.ks[row * Bf16Smem<D>::kStride + col]) = val;
  }
  // V: each thread loads a 4-key x 8-d block (four 16-byte row chunks) and
  // writes it transposed as eight 8-byte runs of 4 keys.  Keys past N are
  // zero so that a masked probability of 0 never meets a non-finite value.
#pragma unroll
  for (int c = tid; c < (kBN / 4) * kChunksPerRow; c += kThreads) {
    const int dg = c % kChunksPerRow;
    const int kg = c / kChunksPerRow;
    u32x4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kv0 + 4 * kg + j;
      r[j] = u32x4{0u, 0u, 0u, 0u};
      if (key < N) r[j] = *reinterpret_cast<const u32x4*>(Vb + (size_t)key * D + 8 * dg);
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int w = cc >> 1;
      const int sh = (cc & 1) * 16;
      const uint32_t e0 = (r[0][w] >> sh) & 0xffffu, e1 = (r[1][w] >> sh) & 0xffffu;
      const uint32_t e2 = (r[2][w] >> sh) & 0xffffu, e3 = (r[3][w] >> sh) & 0xffffu;
      const u32x2 out = {e0 | (e1 << 16), e2 | (e3 << 16)};
      *reinterpret_cast<u32x2*>(&sm.vt[(8 * dg + cc) * Bf16Smem<D>::vStride + 4 * kg]) = out;
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ Lse, int N,
    int num_qtiles, int total_blocks, float scale, float scale_log2) {
  static_assert(D == 64 || D == 128, "head dimension");
  __shared__ Bf16Smem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31;  // query column of this lane inside the wave's 32
  const int hh = lane >> 5;  // half-wave

  const int logical = xcd_remap(blockIdx.x, total_blocks);
  const int bh = logical / num_qtiles;
  int qt = logical - bh * num_qtiles;
  if (CAUSAL) qt = num_qtiles - 1 - qt;  // longest rows first
  const int q0 = qt * kBM;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qb = Q + head;
  const uint16_t* Kb = K + head;
  const uint16_t* Vb = V + head;

  const int wq0 = q0 + wave * 32;  // first query row of this wave
  const int qrow = wq0 + qi;

  // Q^T as the B operand of S^T = K Q^T: lane holds d = 16s + 8hh + (0..7).
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < N) v = *reinterpret_cast<const u32x4*>(Qb + (size_t)qrow * D + 16 * s + 8 * hh);
    qf[s] = __builtin_bit_cast(bf16x8, v);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  // Running state of this lane's query row.  m_run is the largest raw score
  // q.k seen so far; base_run = fl(m_run * scale_log2) is the base-2 reference
  // that every probability and the denominator are taken relative to (kept
  // as the rounded value itself, so that rescaling from one reference to the
  // next, exp2(base_old - base_new), is exact in the exponent).  base_run
  // stays -inf until the row has seen a visible key, making the first
  // rescale factor exactly 0.
  float m_run = kNegInf;
  float base_run = kNegInf;
  float l_run = 0.f;  // this half-wave's part of the denominator

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int arow = key_of_row(qi);

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBN;
    __syncthreads();  // every wave is done with the previous tile
    stage_kv_tile<D>(sm, Kb, Vb, kv0, N, tid);
    __syncthreads();
    if (CAUSAL && kv0 > wq0 + 31) continue;  // the whole tile is above this wave's rows

    // S^T for two 32-key blocks: element 4g+r of block kb is key
    // kv0 + 32kb + key_of_row(8g + 4hh + r) against query qrow.
    f32x16 sacc[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      sacc[kb] = f32x16{};
      const uint16_t* krow = &sm.ks[(32 * kb + arow) * Bf16Smem<D>::kStride + 8 * hh];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_bf16x8(krow + 16 * s),
                                                           qf[s], sacc[kb], 0, 0, 0);
      }
    }

    const bool need_mask = (kv0 + kBN > N) || (CAUSAL && kv0 + kBN - 1 > wq0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + 32 * kb + key_of_row(8 * (e >> 2) + 4 * hh + (e & 3));
          const bool hidden = key >= N || (CAUSAL && key > qrow);
          if (hidden) sacc[kb][e] = kNegInf;
        }
      }
    }

    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx);
    const float base = (m_new == kNegInf) ? 0.f : m_new * scale_log2;
    const float alpha = fast_exp2(base_run - base);
    base_run = (m_new == kNegInf) ? kNegInf : base;

    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(__builtin_fmaf(sacc[kb][e], scale_log2, -base));
        sacc[kb][e] = p;
        lsum += p;
      }
    l_run = alpha * l_run + lsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;

    // P^T as the B operand of O^T += V^T P^T: 16-key step s2 takes elements
    // 8(s2%2) .. 8(s2%2)+7 of score block s2/2, i.e. keys 16 s2 + 8hh + (0..7).
    bf16x8 pf[kBN / 16];
#pragma unroll
    for (int s2 = 0; s2 < kBN / 16; ++s2)
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[s2][j] = (__bf16)sacc[s2 >> 1][8 * (s2 & 1) + j];

#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint16_t* vrow = &sm.vt[(32 * db + qi) * Bf16Smem<D>::vStride + 8 * hh];
#pragma unroll
      for (int s2 = 0; s2 < kBN / 16; ++s2) {
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_bf16x8(vrow + 16 * s2),
                                                           pf[s2], oacc[db], 0, 0, 0);
      }
    }
  }

  // Epilogue: O^T element 4g+r of block db is O[qrow][32db + 8g + 4hh + r].
  const float l_tot = l_run + other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __bf16 o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = (__bf16)(oacc[db][4 * g + r] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * hh) =
            __builtin_bit_cast(u32x2, o4);
      }
    if (hh == 0) {
      // l_tot = sum_j exp2(s_j c - base_run) with base_run = m_run c - r, where
      // r (exact, from one FMA) is the rounding residual of base_run; hence
      // ln sum_j exp(scale s_j) = m_run scale + ln l_tot - r ln 2.
      const float r = __builtin_fmaf(m_run, scale_log2, -base_run);
      Lse[(size_t)bh * N + qrow] =
          l_tot > 0.f ? __builtin_fmaf(m_run, scale, logf(l_tot) - r * kLn2) : kNegInf;
    }
  }
}

}  // namespace fa355
