// Attention forward, bf16 in / bf16 out, fp32 accumulation, on gfx950 MFMA.
//
// Method: the one-pass tiled attention of the wmrh.cn FlashAttention article
// (section 2.2): one workgroup fixes a block of query rows and streams every
// 64-key block of K and V through LDS, keeping per row the running score
// maximum, the softmax denominator l taken relative to a reference point, and
// the un-normalised output.  After the last block the output is divided by l
// once.  Moving the reference point rescales l and the output by
// e^{old - new} (the concatenation rule in the Triton article's section on
// tiled attention).
//
// gfx950 design:
//  * 8 waves x 32 query rows = 256 rows per workgroup, two waves per SIMD, so
//    that one wave's exp/VALU work overlaps the other's MFMA work and every
//    K/V byte fetched from L2 serves 256 rows.
//  * Scores are produced transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane owns one query column, so a row's
//    maximum and sum are in-lane reductions plus one half-wave exchange.
//  * The output is accumulated transposed too, O^T += V^T P^T, with P^T going
//    from the score accumulator into the MFMA B operand in registers; the 32
//    A-operand rows of the score MFMA are mapped to keys by `key_of_row` so
//    that each half-wave holds 8 consecutive keys per 16-key step.
//  * K tiles go from global memory straight into LDS (global_load_lds_dwordx4,
//    no registers), row-major with XOR-swizzled 16-byte chunks.  V tiles go
//    through registers one tile ahead, are transposed in 4x4 blocks with
//    v_perm_b32 and stored as V^T ([d][key]), also swizzled; both are read
//    with conflict-free ds_read_b128.  Both are double-buffered with a single
//    barrier per tile, and K runs one tile ahead of V so that the score MFMAs
//    of tile j+1 are issued before the softmax of tile j.
//  * The reference point of the online softmax moves only when a row's maximum
//    grows by more than 2^8 (in base-2 units); until then probabilities are
//    taken against the stale reference and are at most 2^8, which fp32 and
//    bf16 hold exactly as well.  Softmax is invariant to the shift, so this is
//    the same result while skipping almost every rescale of the output.
//  * Scores are scaled by scale*log2(e) inside one FMA and exponentiated with
//    v_exp_f32 (base 2); L is formed in natural-log units at the end.
#pragma once

#include "fa_common.hpp"

namespace fa355 {

constexpr int kBM = 256;       // query rows per workgroup
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.0f;   // allowed growth of a row maximum before rescaling (log2 units)

template <int D>
struct Bf16Layout {
  static constexpr int kTileBytes = kBN * D * 2;      // one K tile or one V^T tile
  static constexpr int kOffK0 = 0;
  static constexpr int kOffK1 = kTileBytes;
  static constexpr int kOffV0 = 2 * kTileBytes;
  static constexpr int kOffV1 = 3 * kTileBytes;
  static constexpr int kBytes = 4 * kTileBytes;       // 64 KB at d = 128
  static constexpr int kRowBytesK = 2 * D;            // K row: D bf16
  static constexpr int kRowBytesV = 2 * kBN;          // V^T row: kBN bf16
  static constexpr int kKLoadsPerTile = kTileBytes / 1024;  // 1 KB per wave-wide direct load
};

// 16-byte chunk swizzles (chunk index XOR a function of the row) that keep
// both the writes and the MFMA-operand reads of a tile free of LDS bank
// conflicts.  K rows are 2D bytes; V^T rows are 128 bytes.
template <int D>
__device__ __forceinline__ int k_swizzle(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int vt_swizzle(int d) { return ((d >> 1) & 7) ^ ((d >> 4) & 1); }

// Key (within a 32-key block) fed to A-operand row i of the score MFMA.  With
// i = 8g + 4h + r (g = 0..3, h = 0..1, r = 0..3) the accumulator element
// 4g + r of half-wave h holds row i; this mapping makes the elements
// 8s .. 8s+7 of half-wave h equal the keys 16s + 8h + (0..7), s = 0..1.
__device__ __forceinline__ int key_of_row(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + r;
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const char* smem, int byte_off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + byte_off));
}

// Direct global->LDS copy of one K tile.  Each wave issues kKLoadsPerTile/8
// instructions; lane i of an instruction fills physical bytes [16i, 16i+16) of
// its 1 KB slice, so it fetches the logical chunk that the swizzle puts there.
// Rows past N are clamped to row N-1: their scores are masked anyway.
template <int D>
__device__ __forceinline__ void load_k_tile_direct(char* smem, int buf_off,
                                                   const uint16_t* __restrict__ Kb, int kv0,
                                                   int N, int wave, int lane) {
  using Lay = Bf16Layout<D>;
  constexpr int kPerWave = Lay::kKLoadsPerTile / kWaves;
  static_assert(kPerWave >= 1 && Lay::kKLoadsPerTile % kWaves == 0, "K tile split");
#pragma unroll
  for (int r = 0; r < kPerWave; ++r) {
    const int slice = wave * kPerWave + r;
    const int phys = slice * 1024 + 16 * lane;
    const int row = phys / Lay::kRowBytesK;
    const int pch = (phys % Lay::kRowBytesK) / 16;
    const int ch = pch ^ k_swizzle<D>(row);
    const int key = min(kv0 + row, N - 1);
    const uint16_t* src = Kb + (size_t)key * D + 8 * ch;
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<__attribute__((address_space(1))) void*>(reinterpret_cast<uintptr_t>(src)),
        reinterpret_cast<__attribute__((address_space(3))) void*>(
            reinterpret_cast<uintptr_t>(smem + buf_off + slice * 1024)),
        16, 0, 0);
  }
}

// V tile staging through registers: each thread owns 4-key x 4-d blocks.
template <int D>
struct VStage {
  static constexpr int kBlocks = (kBN / 4) * (D / 4);
  static constexpr int kPerThread = (kBlocks + kThreads - 1) / kThreads;
  u32x2 r[kPerThread][4];
};

template <int D>
__device__ __forceinline__ void load_v_tile(VStage<D>& st, const uint16_t* __restrict__ Vb,
                                            int kv0, int N, int tid) {
#pragma unroll
  for (int b = 0; b < VStage<D>::kPerThread; ++b) {
    const int blk = tid + b * kThreads;
    if (VStage<D>::kBlocks % kThreads != 0 && blk >= VStage<D>::kBlocks) break;
    const int dq = blk % (D / 4), kq = blk / (D / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(kv0 + 4 * kq + j, N - 1);  // clamped rows get probability 0
      st.r[b][j] = *reinterpret_cast<const u32x2*>(Vb + (size_t)key * D + 4 * dq);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_vt_tile(char* smem, int buf_off, const VStage<D>& st,
                                              int tid) {
#pragma unroll
  for (int b = 0; b < VStage<D>::kPerThread; ++b) {
    const int blk = tid + b * kThreads;
    if (VStage<D>::kBlocks % kThreads != 0 && blk >= VStage<D>::kBlocks) break;
    const int dq = blk % (D / 4), kq = blk / (D / 4);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // keys 4kq..4kq+3 of component d = 4dq + c, packed two per dword
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      const int w = c >> 1;
      const u32x2 out = {__builtin_amdgcn_perm(st.r[b][1][w], st.r[b][0][w], sel),
                         __builtin_amdgcn_perm(st.r[b][3][w], st.r[b][2][w], sel)};
      const int d = 4 * dq + c;
      const int off = d * Bf16Layout<D>::kRowBytesV + 16 * ((kq >> 1) ^ vt_swizzle(d)) + 8 * (kq & 1);
      *reinterpret_cast<u32x2*>(smem + buf_off + off) = out;
    }
  }
}

__device__ __forceinline__ void wait_vm_and_barrier() {
  // vmcnt(0): direct-to-LDS copies and register loads have landed.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

template <int D>
__device__ __forceinline__ void score_tile(const char* smem, int kbuf, int arow, int hh,
                                           const bf16x8 (&qf)[D / 16], f32x16 (&sacc)[2]) {
  using Lay = Bf16Layout<D>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sacc[kb] = f32x16{};
    const int row = 32 * kb + arow;
    const int rbase = kbuf + row * Lay::kRowBytesK;
    const int sw = k_swizzle<D>(row);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 a = lds_bf16x8(smem, rbase + 16 * ((2 * s + hh) ^ sw));
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ Lse, int N,
    int num_qtiles, int total_blocks, float scale, float scale_log2) {
  static_assert(D == 64 || D == 128, "head dimension");
  using Lay = Bf16Layout<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

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

  // Tiles the workgroup streams, and the prefix of them this wave needs.
  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  int my_tiles = 0;
  if (wq0 < N) {
    const int wave_end = CAUSAL ? min(N, wq0 + 32) : N;
    my_tiles = (wave_end + kBN - 1) / kBN;
  }

  // Q^T as the B operand of S^T = K Q^T: lane holds d = 16s + 8hh + (0..7).
  bf16x8 qf[D / 16];
  {
    const int qr = min(qrow, N - 1);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(Qb + (size_t)qr * D + 16 * s + 8 * hh));
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  // Running state of this lane's query row: base_run is the base-2 reference
  // (a rounded product m_ref * scale_log2, kept as that rounded value so that
  // exp2(base_old - base_new) moves the reference exactly); m_ref is the raw
  // score it came from.  -FLT_MAX marks "no visible key yet".
  float base_run = -__FLT_MAX__;
  float m_ref = kNegInf;
  float l_run = 0.f;  // this half-wave's part of the denominator
  const int arow = key_of_row(qi);

  // Prologue: K_0, K_1 and V_0 into LDS.
  VStage<D> vst;
  load_k_tile_direct<D>(smem, Lay::kOffK0, Kb, 0, N, wave, lane);
  if (n_tiles > 1) load_k_tile_direct<D>(smem, Lay::kOffK1, Kb, kBN, N, wave, lane);
  load_v_tile<D>(vst, Vb, 0, N, tid);
  store_vt_tile<D>(smem, Lay::kOffV0, vst, tid);
  wait_vm_and_barrier();

  f32x16 sacc[2];
  if (my_tiles > 0) score_tile<D>(smem, Lay::kOffK0, arow, hh, qf, sacc);

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBN;
    const int kcur = (t & 1) ? Lay::kOffK1 : Lay::kOffK0;   // holds K_t (consumed)
    const int knext = (t & 1) ? Lay::kOffK0 : Lay::kOffK1;  // holds K_{t+1}
    const int vcur = (t & 1) ? Lay::kOffV1 : Lay::kOffV0;   // holds V_t
    const int vnext = (t & 1) ? Lay::kOffV0 : Lay::kOffV1;  // receives V_{t+1}

    // Prefetch: V_{t+1} into registers, K_{t+2} straight into the buffer K_t left.
    if (t + 1 < n_tiles) load_v_tile<D>(vst, Vb, kv0 + kBN, N, tid);
    if (t + 2 < n_tiles) load_k_tile_direct<D>(smem, kcur, Kb, kv0 + 2 * kBN, N, wave, lane);

    if (t < my_tiles) {
      // Scores of the next tile first, so the MFMAs run under this tile's softmax.
      f32x16 snext[2];
      if (t + 1 < my_tiles) score_tile<D>(smem, knext, arow, hh, qf, snext);

      // sacc element 4g+r of block kb is key kv0 + 32kb + key_of_row(8g + 4hh + r).
      const bool need_mask = (kv0 + kBN > N) || (CAUSAL && kv0 + kBN - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kv0 + 32 * kb + key_of_row(8 * (e >> 2) + 4 * hh + (e & 3));
            if (key >= N || (CAUSAL && key > qrow)) sacc[kb][e] = kNegInf;
          }
      }

      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(sacc[kb][e], sacc[kb][e + 1]));
      mx = fmaxf(mx, other_half(mx));
      const float cand = mx * scale_log2;  // -inf for a fully masked tile
      const bool need = cand > base_run + kTau;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float base_new = need ? cand : base_run;
        const float alpha = fast_exp2(base_run - base_new);
        if (need) m_ref = mx;
        base_run = base_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      }

      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(sacc[kb][e], scale_log2, -base_run));
          sacc[kb][e] = p;
          lsum += p;
        }
      l_run += lsum;

      // P^T as the B operand of O^T += V^T P^T: 16-key step s2 takes elements
      // 8(s2%2) .. 8(s2%2)+7 of score block s2/2, i.e. keys 16 s2 + 8hh + (0..7).
      bf16x8 pf[kBN / 16];
#pragma unroll
      for (int s2 = 0; s2 < kBN / 16; ++s2)
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[s2][j] = (__bf16)sacc[s2 >> 1][8 * (s2 & 1) + j];

#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = 32 * db + qi;
        const int rbase = vcur + d * Lay::kRowBytesV;
        const int sw = vt_swizzle(d);
#pragma unroll
        for (int s2 = 0; s2 < kBN / 16; ++s2) {
          const bf16x8 a = lds_bf16x8(smem, rbase + 16 * ((2 * s2 + hh) ^ sw));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s2], oacc[db], 0, 0, 0);
        }
      }
      sacc[0] = snext[0];
      sacc[1] = snext[1];
    }

    if (t + 1 < n_tiles) store_vt_tile<D>(smem, vnext, vst, tid);
    wait_vm_and_barrier();
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
      // l_tot = sum_j exp2(s_j c - base_run) with base_run = m_ref c - r, where
      // r (exact, from one FMA) is the rounding residual of base_run; hence
      // ln sum_j exp(scale s_j) = m_ref scale + ln l_tot - r ln 2.
      const float r = __builtin_fmaf(m_ref, scale_log2, -base_run);
      Lse[(size_t)bh * N + qrow] =
          l_tot > 0.f ? __builtin_fmaf(m_ref, scale, logf(l_tot) - r * kLn2) : kNegInf;
    }
  }
}

}  // namespace fa355
