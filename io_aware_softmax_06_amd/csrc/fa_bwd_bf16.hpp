// Attention backward, bf16 in / bf16 out, fp32 accumulation, on gfx950 MFMA.
//
// The gradients of <dO, O> recompute the score matrix from Q, K and the
// forward's logsumexp L instead of storing it (the Triton article's section
// on the core idea, 核心思想).  With P = exp(scale S - L) (hidden scores 0):
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_d dO_id O_id,
//     dQ = scale dS K,  dK = scale dS^T Q.
// D_i equals sum_j P_ij dP_ij because O = P V; it is computed once per row
// by fa_bwd_dot_kernel.
//
// Two kernels, so that no result is accumulated across workgroups (no
// atomics; the output is deterministic):
//  * fa_bwd_dkdv_bf16_kernel: a workgroup owns 128 keys and streams the
//    query tiles of its head; K and V sit in registers as the B operands of
//    S = Q K^T and dP = dO V^T (one key per lane), and dV^T and dK^T
//    accumulate from P and dS taken straight from those accumulators, in two
//    waves per 32 keys (one per product).
//  * fa_bwd_dq_bf16_kernel: a workgroup owns 256 queries (8 waves x 32) and
//    streams the key tiles, like the forward: S^T = K Q^T and dP^T = V dO^T
//    with one query per lane, then dQ^T += K^T dS^T.
// Both reuse the forward's operand reads (score_tile, pv_tile) and tile
// layouts: a tile whose rows are the MFMA A operand is stored K-style, a
// tile read transposed (K^T, Q^T, dO^T) V-style.  Tiles are double buffered
// with one barrier per tile.
#pragma once

#include <type_traits>

#include "fa_fwd_bf16.hpp"

namespace FA355_NS {

// ---------------------------------------------------------------------------
// D_i = sum_d dO_id O_id in float32, one row per D/8 threads.
constexpr int kDotThreads = 256;

__device__ __forceinline__ void load8(const __bf16* p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const _Float16* p, float (&x)[8]) {
  const f16x8 w = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)w[i];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

template <int D, typename T>
__global__ __launch_bounds__(kDotThreads) void fa_bwd_dot_kernel(const T* __restrict__ O,
                                                                 const T* __restrict__ dO,
                                                                 float* __restrict__ Dv,
                                                                 int64_t rows) {
  constexpr int kPer = D / 8;  // threads per row: 4, 8 or 16, a power of two inside one wave
  constexpr int kRowsPer = kDotThreads / kPer;
  const int c = threadIdx.x % kPer;
  const int64_t stride = (int64_t)gridDim.x * kRowsPer;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPer + threadIdx.x / kPer; row < rows;
       row += stride) {
    float o[8], g[8];
    load8(O + row * D + 8 * c, o);
    load8(dO + row * D + 8 * c, g);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(o[i], g[i], acc);
#pragma unroll
    for (int off = kPer / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (c == 0) Dv[row] = acc;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two bf16 kernels.

// bf16 B operand of a 32-row MFMA column: elements 16s + 8hh + (0..7) of row
// `row` (a key of K or V, or a query of Q or dO), s = 0 .. D/16 - 1.
template <int D, typename V8>
__device__ __forceinline__ void load_b_operand(const uint16_t* __restrict__ head, int row, int hh,
                                               V8 (&f)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    f[s] = __builtin_bit_cast(V8,
                              *reinterpret_cast<const u32x4*>(head + (size_t)row * D + 16 * s + 8 * hh));
}

// 16-key (or 16-query) step s2 of a 32x64 accumulator pair as a bf16 B operand.
template <typename T>
__device__ __forceinline__ void to_b_operand(const f32x16 (&x)[2],
                                             typename Elem<T>::v8 (&f)[kBN / 16]) {
#pragma unroll
  for (int s2 = 0; s2 < kBN / 16; ++s2)
#pragma unroll
    for (int j = 0; j < 8; ++j) f[s2][j] = (T)x[s2 >> 1][8 * (s2 & 1) + j];
}

// Store a transposed accumulator (lane = row of the output, element 4g+r of
// block db = column 32db + 8g + 4hh + r) times `mul` as bf16.
template <int D, typename T>
__device__ __forceinline__ void store_rows(uint16_t* __restrict__ out_row, const f32x16 (&acc)[D / 32],
                                          float mul, int hh) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      T o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = (T)(acc[db][4 * g + r] * mul);
      *reinterpret_cast<u32x2*>(out_row + 32 * db + 8 * g + 4 * hh) = __builtin_bit_cast(u32x2, o4);
    }
}

// p * t with p a float16 taken from the low (H = 0) or high (H = 1) half of a
// packed pair and t a float32: one v_fma_mix_f32 (p converted exactly, plus
// 0) instead of a conversion and a multiply.
template <int H>
__device__ __forceinline__ float mul_f16_f32(uint32_t p2, float t) {
  float r;
  if constexpr (H == 0)
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(p2), "v"(t));
  else
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(p2), "v"(t));
  return r;
}

// 64 floats (one per row of a tile) straight into LDS; rows past the end of
// the resource read as 0.  Issued by one wave.
__device__ __forceinline__ void load_row_floats(char* smem, int off, __amdgpu_buffer_rsrc_t rsrc,
                                                int row0, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc,
      reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(smem + off)),
      4, (uint32_t)(row0 + lane) * 4u, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (batch*head, 128 keys), 8 waves in two roles.
// Waves w and w + 4 share a SIMD and own the same 32 keys (key block w % 4).
// Per query tile the dV wave forms S = Q K^T and P, and the dK wave forms
// dP = dO V^T; the dV wave hands P (as float16) to the dK wave through LDS,
// and after a barrier the dV wave accumulates dV^T += dO^T P while the dK
// wave forms dS = P (dP - D) and accumulates dK^T += Q^T dS.  Each wave holds
// half the operands and accumulators of one wave doing both products, so
// that two waves fit on a SIMD and one wave's exponentials and conversions
// run under the other's MFMAs.
constexpr int kBwdKvWaves = 8;
constexpr int kBwdKvKeys = 32 * (kBwdKvWaves / 2);

template <int D>
struct BwdKvLayout {
  static constexpr int kTile = Bf16Layout<D>::kTileBytes;  // 64 rows x D bf16
  static constexpr int kOffQk = 0, kOffDok = kTile, kOffQv = 2 * kTile, kOffDov = 3 * kTile;
  static constexpr int kOffL = 4 * kTile, kOffD = 4 * kTile + 256;
  static constexpr int kStage = 4 * kTile + 512;
  // P of the current tile, one 4 KB slot per key block: lane l's 16-key step
  // s2 (eight float16) at byte (s2 * 64 + l) * 16 of its block's slot.
  static constexpr int kOffP = 2 * kStage, kPSlot = 64 * 64;
  static constexpr int kBytes = 2 * kStage + (kBwdKvWaves / 2) * kPSlot;
  static_assert(kBytes <= 160 * 1024, "LDS per workgroup");
};

template <int D, bool CAUSAL, typename T = __bf16>
__global__ __launch_bounds__(64 * kBwdKvWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void
fa_bwd_dkdv_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                        const float* __restrict__ Lse, const float* __restrict__ Dv,
                        uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int BH,
                        float scale, float scale_log2) {
  static_assert(D == 32 || D == 64 || D == 128, "head dimension");
  using Lay = BwdKvLayout<D>;
  using V8 = typename Elem<T>::v8;
  constexpr int W = kBwdKvWaves;
  constexpr int kPer = Bf16Layout<D>::kLoadsPerTile >= W ? Bf16Layout<D>::kLoadsPerTile / W : 1;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31, hh = lane >> 5;
  // The role is the same in every lane: take it from a scalar register so
  // that the branch below is a scalar branch.
  const bool dk_role = __builtin_amdgcn_readfirstlane(wave) >= W / 2;
  const int kblk = wave & (W / 2 - 1);

  // Workgroup -> (head, key block).  Heads stay whole on one XCD; with the
  // causal mask the first key blocks see the most queries, so they go first
  // (key block outermost: measured 4% faster than finishing a head's blocks
  // before the next head's, despite the wider working set in L2).
  const int nk = (N + kBwdKvKeys - 1) / kBwdKvKeys;
  int bh, kt;
  {
    constexpr int kXcds = 8;
    const int bid = blockIdx.x;
    if (BH % kXcds == 0) {
      const int hp = BH / kXcds, xcd = bid % kXcds, slot = bid / kXcds;
      if (CAUSAL) {
        kt = slot / hp;
        bh = xcd * hp + slot % hp;
      } else {
        bh = xcd * hp + slot / nk;
        kt = slot % nk;
      }
    } else if (CAUSAL) {
      kt = bid / BH;
      bh = bid % BH;
    } else {
      bh = bid / nk;
      kt = bid % nk;
    }
  }
  const int k0 = kt * kBwdKvKeys;
  const int kw0 = k0 + 32 * kblk;  // first key of this wave
  const int key = kw0 + qi;        // this lane's key
  const size_t head = (size_t)bh * N * D;

  // Query tiles: with the causal mask only those that reach this workgroup's
  // first key.
  const int nq = (N + kBN - 1) / kBN;
  const int t0 = CAUSAL ? k0 / kBN : 0;

  const int arow = key_of_row(qi);
  const int k_lane = arow * 32 + 16 * (hh ^ ((arow >> 3) & 1));
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_lane = (8 * (g16 >> 1) + (j16 >> 2)) * 64 + 2 * (16 * (g16 & 1) + 4 * (j16 & 3));
  const uint32_t smem_lds = lds_address(smem);
  uint32_t k_off[kPer], v_off[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    k_off[r] = tile_lane_offset<D, false, W>(wave, lane, r);
    v_off[r] = tile_lane_offset<D, true, W>(wave, lane, r);
  }
  const __amdgpu_buffer_rsrc_t q_rsrc = head_resource(Q + head, N * D * 2);
  const __amdgpu_buffer_rsrc_t do_rsrc = head_resource(dO + head, N * D * 2);
  const __amdgpu_buffer_rsrc_t l_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(Lse + (size_t)bh * N), (short)0, N * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t d_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(Dv + (size_t)bh * N), (short)0, N * 4, kBufferWord3);
  // This lane's 16-byte pieces of its key block's P slot.
  u32x4* p_slot = reinterpret_cast<u32x4*>(smem + Lay::kOffP + kblk * Lay::kPSlot) + lane;

  // Every wave issues its share of every tile: Q and dO both K-style (rows as
  // A operands) and V-style (read transposed), plus L and D.  The V-style Q
  // goes separately (load_qv): the dK wave reads it one iteration late.
  auto load_main = [&](int t) {
    const int st = (t & 1) * Lay::kStage, q0 = t * kBN;
    load_tile_direct<D, W>(smem, st + Lay::kOffQk, q_rsrc, q0, wave, k_off);
    load_tile_direct<D, W>(smem, st + Lay::kOffDok, do_rsrc, q0, wave, k_off);
    load_tile_direct<D, W>(smem, st + Lay::kOffDov, do_rsrc, q0, wave, v_off);
    if (wave == 0) {
      load_row_floats(smem, st + Lay::kOffL, l_rsrc, q0, lane);
      load_row_floats(smem, st + Lay::kOffD, d_rsrc, q0, lane);
    }
  };
  auto load_qv = [&](int t) {
    load_tile_direct<D, W>(smem, (t & 1) * Lay::kStage + Lay::kOffQv, q_rsrc, t * kBN, wave,
                           v_off);
  };

  // One role's loop: K^T (dV role) or V^T (dK role) as the B operand of its
  // score-shaped product, one key per lane, fixed for the workgroup; the
  // role's accumulator; two barriers per tile.  Every wave passes every
  // barrier, also on tiles its keys do not see.
  //
  // Software pipeline of the dK wave: it forms dS of tile t after the second
  // barrier and accumulates Q_t^T dS_t only in the first half of iteration
  // t+1, under the dV wave's exponentials.  So the V-style Q_t must stay
  // until the second barrier of iteration t+1: it is loaded after the second
  // barrier of iteration t-1 (into the stage of tile t-1, whose V-style Q the
  // dK wave has just used), and the wait at the top of an iteration lets that
  // one load stay in flight.
  auto run = [&](auto dk_ic) {
    constexpr bool DK = decltype(dk_ic)::value;
    V8 bop[D / 16];
    load_b_operand<D>((DK ? V : K) + head, min(key, N - 1), hh, bop);
    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
    V8 bf[kBN / 16];    // P (dV role) or dS (dK role) as B operands
    bool held = false;  // dK role: bf holds dS of the previous tile

    if (t0 < nq) {
      load_main(t0);
      load_qv(t0);
    }
    for (int t = t0; t < nq; ++t) {
      // Tile t has landed for every wave, and so has the V-style Q of tile
      // t-1; only tile t's own V-style Q may be in flight.  Tile t-1's stage
      // is free except for its V-style Q, and so is the P slot (the dK wave
      // read P_{t-1} before this barrier).
      wait_vmcnt<kPer>();
      if (wave == 0) {
        // The tile's L becomes the exponent offset -L log2(e) once, here,
        // instead of in every dV lane for every element (-inf, a row that
        // saw no key, stays -inf so that its probabilities are 0).
        float* lt = reinterpret_cast<float*>(smem + (t & 1) * Lay::kStage + Lay::kOffL) + lane;
        const float l = *lt;
        *lt = l == kNegInf ? kNegInf : -l * kLog2e;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      block_sync();
      if (t + 1 < nq) load_main(t + 1);
      const int q0 = t * kBN;
      // A wave whose keys all lie after the tile's last query has nothing to do
      // (the same in every lane: a scalar, so that the branches on it are).
      const bool active =
          __builtin_amdgcn_readfirstlane((kw0 < N && !(CAUSAL && q0 + kBN - 1 < kw0)) ? 1 : 0) != 0;
      const uint32_t st = smem_lds + (t & 1) * Lay::kStage;
      const char* stage = smem + (t & 1) * Lay::kStage;

      // S[q][key] (dV role) or dP[q][key] (dK role): element 4g+r of block kb
      // is query q0 + 32kb + key_of_row(8g + 4hh + r).
      f32x16 sacc[2];
      if (active) {
        score_tile<D, T>(st + (DK ? Lay::kOffDok : Lay::kOffQk) + k_lane, bop, sacc);
        if constexpr (!DK) {
          // P = exp(scale S - L); the four queries of a group g are
          // consecutive, so their offsets -L log2(e) come as one 16-byte read.
          const float* Lt = reinterpret_cast<const float*>(stage + Lay::kOffL);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int qoff = 32 * kb + 16 * (g >> 1) + 8 * hh + 4 * (g & 1);
              const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + qoff);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                sacc[kb][4 * g + r] =
                    fast_exp2(__builtin_fmaf(sacc[kb][4 * g + r], scale_log2, l4[r]));
            }
          // Only tiles on the diagonal or past N need the mask (a scalar branch).
          const bool need_mask =
              __builtin_amdgcn_readfirstlane(((q0 + kBN > N) || (CAUSAL && kw0 + 31 > q0)) ? 1 : 0) != 0;
          if (need_mask) {
            // (kept a real branch: without it the masking is folded into
            // selects that every tile pays for)
            asm volatile("" ::: "memory");
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int q = q0 + 32 * kb + 16 * (e >> 3) + 8 * hh + 4 * ((e >> 2) & 1) + (e & 3);
                if (q >= N || (CAUSAL && key > q)) sacc[kb][e] = 0.f;
              }
          }
          to_b_operand<T>(sacc, bf);
          // P goes to the dK wave as float16 whatever the input type: P <= 1,
          // and float16 keeps 11 bits of it (bfloat16 8), so dS loses nothing
          // measurable against a float32 P.
          f16x8 ph[kBN / 16];
          if constexpr (std::is_same<T, _Float16>::value) {
#pragma unroll
            for (int s2 = 0; s2 < kBN / 16; ++s2) ph[s2] = __builtin_bit_cast(f16x8, bf[s2]);
          } else {
            to_b_operand<_Float16>(sacc, ph);
          }
#pragma unroll
          for (int s2 = 0; s2 < kBN / 16; ++s2)
            p_slot[64 * s2] = __builtin_bit_cast(u32x4, ph[s2]);
          // P is in LDS before this wave reaches the barrier (the clobber
          // keeps the stores above the wait).
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
      }
      if constexpr (DK) {
        // dK^T += Q_{t-1}^T dS_{t-1} (lane = key), from the previous stage.
        if (held)
          pv_tile<D, T>(smem_lds + ((t - 1) & 1) * Lay::kStage + Lay::kOffQv + v_lane, bf, acc);
        held = false;
      }
      block_sync();  // P of tile t is in LDS; the V-style Q of tile t-1 is read
      if (t + 1 < nq) load_qv(t + 1);
      if (!active) continue;
      if constexpr (DK) {
        // dS = P (dP - D), with P from the dV wave (float16).
        const float* Dt = reinterpret_cast<const float*>(stage + Lay::kOffD);
        u32x4 pp[kBN / 16];  // eight float16 per 16-key step, as four packed pairs
#pragma unroll
        for (int s2 = 0; s2 < kBN / 16; ++s2) pp[s2] = p_slot[64 * s2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int qoff = 32 * kb + 16 * (g >> 1) + 8 * hh + 4 * (g & 1);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dt + qoff);
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const int e = 4 * g + r;  // elements e, e + 1: one packed pair of P
              const uint32_t p2 = pp[2 * kb + (e >> 3)][(e & 7) >> 1];
              sacc[kb][e] = mul_f16_f32<0>(p2, sacc[kb][e] - d4[r]);
              sacc[kb][e + 1] = mul_f16_f32<1>(p2, sacc[kb][e + 1] - d4[r + 1]);
            }
          }
        to_b_operand<T>(sacc, bf);
        held = true;
      } else {
        // dV^T += dO^T P (lane = key).
        pv_tile<D, T>(st + Lay::kOffDov + v_lane, bf, acc);
      }
    }
    // The last tile's V-style Q: every wave's share has landed before the
    // dK wave reads it.
    wait_vmcnt<0>();
    block_sync();
    if constexpr (DK) {
      if (held)
        pv_tile<D, T>(smem_lds + ((nq - 1) & 1) * Lay::kStage + Lay::kOffQv + v_lane, bf, acc);
    }

    if (key < N) {
      if constexpr (DK) store_rows<D, T>(dK + head + (size_t)key * D, acc, scale, hh);
      else store_rows<D, T>(dV + head + (size_t)key * D, acc, 1.f, hh);
    }
  };
  if (dk_role) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (batch*head, 256 queries), 8 waves x 32 queries.
template <int D>
struct BwdQLayout {
  static constexpr int kTile = Bf16Layout<D>::kTileBytes;
  static constexpr int kOffKk = 0, kOffVk = kTile, kOffKv = 2 * kTile;
  static constexpr int kStage = 3 * kTile;
  static constexpr int kBytes = 2 * kStage;
  static_assert(kBytes <= 160 * 1024, "LDS per workgroup");
};

template <int D, bool CAUSAL, typename T = __bf16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
fa_bwd_dq_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                      const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                      const float* __restrict__ Lse, const float* __restrict__ Dv,
                      uint16_t* __restrict__ dQ, int N, int BH, int num_qtiles, float scale,
                      float scale_log2) {
  static_assert(D == 32 || D == 64 || D == 128, "head dimension");
  using Lay = BwdQLayout<D>;
  using V8 = typename Elem<T>::v8;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31, hh = lane >> 5;

  int bh, qt;
  map_tile<CAUSAL>(blockIdx.x, BH, num_qtiles, bh, qt);
  const int q0 = qt * kBM;
  const int wq0 = q0 + 32 * wave;
  const int qrow = wq0 + qi;
  const size_t head = (size_t)bh * N * D;

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  int my_tiles = 0;
  if (wq0 < N) my_tiles = ((CAUSAL ? min(N, wq0 + 32) : N) + kBN - 1) / kBN;
  my_tiles = __builtin_amdgcn_readfirstlane(my_tiles);  // the same in every lane

  // Q^T and dO^T as B operands (one query per lane); this row's L and D.
  V8 qf[D / 16], dof[D / 16];
  const int qr = min(qrow, N - 1);
  load_b_operand<D>(Q + head, qr, hh, qf);
  load_b_operand<D>(dO + head, qr, hh, dof);
  const float lq = Lse[(size_t)bh * N + qr];
  const float nl = lq == kNegInf ? kNegInf : -lq * kLog2e;
  const float dq_row = Dv[(size_t)bh * N + qr];

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{};

  const int arow = key_of_row(qi);
  const int k_lane = arow * 32 + 16 * (hh ^ ((arow >> 3) & 1));
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_lane = (8 * (g16 >> 1) + (j16 >> 2)) * 64 + 2 * (16 * (g16 & 1) + 4 * (j16 & 3));
  const uint32_t smem_lds = lds_address(smem);
  constexpr int kPer = Bf16Layout<D>::kLoadsPerWave;
  uint32_t k_off[kPer], v_off[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    k_off[r] = tile_lane_offset<D, false>(wave, lane, r);
    v_off[r] = tile_lane_offset<D, true>(wave, lane, r);
  }
  const __amdgpu_buffer_rsrc_t k_rsrc = head_resource(K + head, N * D * 2);
  const __amdgpu_buffer_rsrc_t v_rsrc = head_resource(V + head, N * D * 2);

  auto load_tile = [&](int j) {
    const int st = (j & 1) * Lay::kStage, kv0 = j * kBN;
    load_tile_direct<D>(smem, st + Lay::kOffKk, k_rsrc, kv0, wave, k_off);
    load_tile_direct<D>(smem, st + Lay::kOffVk, v_rsrc, kv0, wave, k_off);
    load_tile_direct<D>(smem, st + Lay::kOffKv, k_rsrc, kv0, wave, v_off);
  };

  if (n_tiles > 0) load_tile(0);
  for (int j = 0; j < n_tiles; ++j) {
    wait_vmcnt<0>();
    block_sync();
    if (j + 1 < n_tiles) load_tile(j + 1);
    if (j >= my_tiles) continue;
    const int kv0 = j * kBN;
    const uint32_t st = smem_lds + (j & 1) * Lay::kStage;

    // S^T[key][q] and dP^T[key][q]: element 4g+r of block kb is key
    // kv0 + 32kb + key_of_row(8g + 4hh + r); lane = query.
    f32x16 sacc[2], dpacc[2];
    score_tile<D, T>(st + Lay::kOffKk + k_lane, qf, sacc);
    score_tile<D, T>(st + Lay::kOffVk + k_lane, dof, dpacc);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = fast_exp2(__builtin_fmaf(sacc[kb][e], scale_log2, nl));
    // Only tiles on the diagonal or past N need the mask: a scalar branch
    // (kept a real one, not folded into selects that every tile would pay).
    const bool need_mask = __builtin_amdgcn_readfirstlane(
                               ((kv0 + kBN > N) || (CAUSAL && kv0 + kBN - 1 > wq0)) ? 1 : 0) != 0;
    if (need_mask) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = kv0 + 32 * kb + key_of_row(8 * (e >> 2) + 4 * hh + (e & 3));
          if (kk >= N || (CAUSAL && kk > qrow)) sacc[kb][e] = 0.f;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) dpacc[kb][e] = sacc[kb][e] * (dpacc[kb][e] - dq_row);
    V8 dsf[kBN / 16];
    to_b_operand<T>(dpacc, dsf);
    // dQ^T += K^T dS^T (K read transposed from its V-style copy).
    pv_tile<D, T>(st + Lay::kOffKv + v_lane, dsf, dqacc);
  }

  if (qrow < N) store_rows<D, T>(dQ + head + (size_t)qrow * D, dqacc, scale, hh);
}

}  // namespace FA355_NS
