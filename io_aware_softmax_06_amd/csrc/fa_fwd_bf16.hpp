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
//    maximum and sum are in-lane reductions plus one half-wave exchange
//    (v_permlane32_swap).
//  * The output is accumulated transposed too, O^T += V^T P^T, with P^T going
//    from the score accumulator into the MFMA B operand in registers; the 32
//    A-operand rows of the score MFMA are mapped to keys by `key_of_row` so
//    that each half-wave holds 8 consecutive keys per 16-key step.
//  * K and V tiles go from global memory straight into LDS
//    (global_load_lds_dwordx4, no registers) in a ring of three buffers each,
//    each tile issued two loop iterations before the one that reads it.  The
//    LDS layouts are cut so that every operand read of a lane is one base
//    register plus a compile-time offset and no read has bank conflicts: K
//    is stored in 32-byte column slabs (one per 16-wide step of d), V in
//    64-byte column slabs (one per 32-wide block of d).  K rows are read as
//    MFMA A operands with ds_read_b128; V^T operands
//    come from the V slabs through ds_read_b64_tr_b16, whose 16-lane transpose
//    turns four 8-byte row pieces into one column fragment.
//  * The softmax VALU work of a tile is split over both MFMA streams of the
//    loop so that every MFMA has VALU work to hide: iteration j runs the
//    P V MFMAs of tile j under the mask, row maximum, reference update and
//    first half of the exponentials of tile j+1, then the score MFMAs of tile
//    j+2 under the second half of those exponentials, the row sums and the
//    bf16 conversion.  sched_group_barrier interleaves each pair; the operand
//    reads are issued a few MFMAs ahead from inline asm.  One barrier per tile.
//  * Causal launches with more query tiles than CUs are persistent: one
//    workgroup per CU walks a balanced list of query tiles, and the K/V ring
//    runs on from one tile to the next, so that the next tile's first K and V
//    tiles load under the current tile's last iterations.
//  * The reference point of the online softmax moves only when a row's maximum
//    grows by more than 8 (in base-2 units); until then probabilities are
//    taken against the stale reference and are at most 2^8 (2^16 on tiles
//    that skip the row maximum, see FastState), which fp32 and bf16 hold as
//    well.  Softmax is invariant to the shift, so this is the same result
//    while skipping almost every rescale of the output.
//  * Scores are scaled by scale*log2(e) inside one FMA and exponentiated with
//    v_exp_f32 (base 2); L is formed in natural-log units at the end.
#pragma once

#include <utility>

#include "fa_common.hpp"

namespace FA355_NS {

#ifndef FA355_BF16_WAVES
#define FA355_BF16_WAVES 8
#endif
#ifndef FA355_BF16_STAGES
#define FA355_BF16_STAGES 3
#endif
#ifndef FA355_BF16_VSTAGES
#define FA355_BF16_VSTAGES FA355_BF16_STAGES
#endif
// 1: the output staging area of every wave sits past the K and V rings (the
// 8-wave build: 160 KB of LDS at d = 128); 0: it reuses the ring memory after
// the last loads (builds that must stay within a smaller LDS footprint).
#ifndef FA355_STAGE_DEDICATED
#define FA355_STAGE_DEDICATED 1
#endif
// Waves of one workgroup per SIMD that the register allocation must allow:
// 2 for the 8-wave workgroups (two per SIMD); 1 when a 4-wave workgroup
// fills the LDS alone (d = 256), which leaves it 512 registers per lane.
#ifndef FA355_BF16_OCCUPANCY
#define FA355_BF16_OCCUPANCY 2
#endif
constexpr int kWaves = FA355_BF16_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup (32 per wave)
constexpr int kBN = 64;           // keys per K/V tile
constexpr int kStages = FA355_BF16_STAGES;    // ring depth of the K tile buffers
constexpr int kVStages = FA355_BF16_VSTAGES;  // ring depth of the V tile buffers
// The loop reads K two tiles ahead of V.  Either both rings are kStages >= 3
// deep, or K is 3 deep and V 2 deep (each V tile then loads during the one
// iteration before it is read).
static_assert((kStages >= 3 && kVStages == kStages) || (kStages == 3 && kVStages == 2),
              "ring depths");
static_assert(kWaves == 4 || kWaves == 8, "waves per workgroup");
constexpr float kTau = 8.0f;   // allowed growth of a row maximum before rescaling (log2 units)
// Score-operand reads issued this many MFMAs ahead of their use.
#ifndef FA355_SCORE_AHEAD
#define FA355_SCORE_AHEAD 4
#endif
#ifndef FA355_XPHASE
#define FA355_XPHASE 1
#endif
constexpr bool kXPhase = FA355_XPHASE;  // score operands prefetched across the phase boundary

// LDS image of one tile (64 keys x D, bf16):
//   K: D/16 slabs of [64 rows][32 bytes] (d = 16s .. 16s+15 of every key), the
//      two 16-byte halves of row r swapped when bit 3 of r is set;
//   V: D/32 slabs of [64 rows][64 bytes] (d = 32db .. 32db+31 of every key).
template <int D>
struct Bf16Layout {
  static constexpr int kTileBytes = kBN * D * 2;      // one K or V tile
  static constexpr int kKSlab = kBN * 32;             // 2 KB
  static constexpr int kVSlab = kBN * 64;             // 4 KB
  static constexpr int kOffK = 0;                     // kStages K tiles
  static constexpr int kOffV = kStages * kTileBytes;  // kVStages V tiles
  static constexpr int kBytes = (kStages + kVStages) * kTileBytes;  // 16 KB per slot at d = 128
  static_assert(kBytes <= 160 * 1024, "LDS per workgroup");
  // Output staging: each wave turns its 32 x D tile of O from column layout
  // (one query per lane) into whole rows in LDS, so that the stores write
  // complete rows.  Rows of D * 2 bytes, 16-byte chunks XOR-swizzled by the
  // row.  Dedicated builds keep the staging area past the rings (no barrier,
  // and the rings may hold the next query tile's first K and V tiles);
  // otherwise it reuses the ring memory once every load has landed.
  static constexpr int kStageRow = D * 2;
  static constexpr int kStageWave = 32 * kStageRow;
  static constexpr int kStageOff = FA355_STAGE_DEDICATED ? kBytes : 0;
  static constexpr int kBytesStaged = FA355_STAGE_DEDICATED ? kBytes + kWaves * kStageWave : kBytes;
  static_assert(kBytesStaged <= 160 * 1024 && kWaves * kStageWave <= kBytes + (kBytesStaged - kBytes),
                "LDS for the output staging");
  static constexpr int kLoadsPerTile = kTileBytes / 1024;  // 1 KB per wave-wide direct load
  // Loads per wave; at d = 32 a tile is 4 KB, fewer pieces than waves, and
  // only the first kLoadsPerTile waves load (one piece each).
  static constexpr int kLoadsPerWave = kLoadsPerTile >= kWaves ? kLoadsPerTile / kWaves : 1;
  static_assert(kLoadsPerTile % kWaves == 0 || kWaves % kLoadsPerTile == 0, "tile split over waves");
};

// Key (within a 32-key block) fed to A-operand row i of the score MFMA.  With
// i = 8g + 4h + r (g = 0..3, h = 0..1, r = 0..3) the accumulator element
// 4g + r of half-wave h holds row i; this mapping makes the elements
// 8s .. 8s+7 of half-wave h equal the keys 16s + 8h + (0..7), s = 0..1.
__device__ __forceinline__ int key_of_row(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * h + 4 * (g & 1) + r;
}

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, with i usable as a constant.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t lds_address(const char* p) {
  // generic -> LDS address-space cast; the LDS pointer's value is the offset
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// i receives element (i % 4) of the 8-byte pieces that lanes 4e + i/4 point
// at, e = 0..3.  Issued from inline asm: the compiler would otherwise wait for
// every outstanding direct-to-LDS load before it, which defeats the prefetch.
// The caller waits for the result with lds_wait<N>() and pins it with pin().
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr16(uint32_t lds_addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "n"(OFF));
  return v;
}
// Plain 16-byte LDS read, issued from inline asm so that its place among the
// other operand reads is fixed (see lds_tr16).
template <int OFF>
__device__ __forceinline__ u32x4 lds_read128(uint32_t lds_addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "n"(OFF));
  return v;
}
template <int N>
__device__ __forceinline__ void lds_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// Orders every later use of v after the preceding lds_wait (asm statements
// keep their relative order; the use depends on this one's output).
__device__ __forceinline__ void pin(u32x2& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(u32x4& v) { asm volatile("" : "+v"(v)); }

// Workgroup barrier without the memory fence of __syncthreads(), whose
// implied vmcnt(0) would also wait for the loads that are meant to stay in
// flight across it.  The callers wait for exactly the loads they need first,
// and every LDS read before it has been consumed (waited for) already.
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their
// maxima).  gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Direct global->LDS copy of one K or V tile through a buffer resource.
// Each wave issues kLoadsPerWave buffer_load_dwordx4 ... lds instructions;
// lane l of instruction (slice) i fills bytes [16l, 16l+16) of the tile's
// i-th kilobyte and fetches the 16 bytes of K or V that the layout puts
// there.  One resource per head covers exactly its N rows and is built once;
// the per-lane byte offset is a loop constant plus the tile's offset, and the
// hardware range check on that offset returns zeros for rows past N (their
// scores are masked and their probabilities are 0), so no row is clamped.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_resource(const uint16_t* head, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(head), (short)0, bytes,
                                           kBufferWord3);
}

template <int D, bool IS_V, int W = kWaves>
__device__ __forceinline__ uint32_t tile_lane_offset(int wave, int lane, int r) {
  using Lay = Bf16Layout<D>;
  constexpr int kPer = Lay::kLoadsPerTile >= W ? Lay::kLoadsPerTile / W : 1;
  const int slice = min(wave * kPer + r, Lay::kLoadsPerTile - 1);  // waves that load nothing
  int row, col;
  if (IS_V) {  // slab db = slice / 4 holds rows 16 (slice % 4) .. +15
    row = 16 * (slice & 3) + (lane >> 2);
    col = 32 * (slice >> 2) + 8 * (lane & 3);
  } else {     // slab s = slice / 2 holds rows 32 (slice % 2) .. +31
    row = 32 * (slice & 1) + (lane >> 1);
    col = 16 * (slice >> 1) + 8 * ((lane & 1) ^ ((row >> 3) & 1));
  }
  return (uint32_t)(row * D + col) * 2u;
}

// rsrc: the head's K or V (head_resource); kv0: first row of the tile; the
// lane offsets come from tile_lane_offset; W waves share the tile's loads.
template <int D, int W = kWaves>
__device__ __forceinline__ void load_tile_direct(char* smem, int buf_off,
                                                 __amdgpu_buffer_rsrc_t rsrc, int kv0, int wave,
                                                 const uint32_t* lane_off) {
  using Lay = Bf16Layout<D>;
  constexpr int kPer = Lay::kLoadsPerTile >= W ? Lay::kLoadsPerTile / W : 1;
  static_assert(Lay::kLoadsPerTile % W == 0 || W % Lay::kLoadsPerTile == 0, "tile split over waves");
  if (Lay::kLoadsPerTile < W && wave >= Lay::kLoadsPerTile) return;  // (uniform per wave)
  const uint32_t tile_off = (uint32_t)kv0 * (D * 2);
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int slice = wave * kPer + r;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc,
        reinterpret_cast<__attribute__((address_space(3))) void*>(
            reinterpret_cast<uintptr_t>(smem + buf_off + slice * 1024)),
        16, lane_off[r] + tile_off, 0, 0, 0);
  }
}

// Scores of one tile, transposed: sacc[kb] = K[32kb + key_of_row(.)] Q^T.
// kaddr = LDS address of this lane's K piece in slab 0, block 0: row
// key_of_row(qi), half hh (swapped by the row's bit 3); slab s and block kb add
// constants.  The operand reads run kAhead MFMAs ahead of their use, in a
// rotation of kAhead + 2 register slots (a slot is refilled two MFMAs after
// the one that read it).  work(i) (VALU work given as an integral constant
// index) follows MFMA i, and a scheduling barrier closes each such chunk, so
// the program order of MFMAs and VALU work is the one written here.
struct NoWork {
  template <typename I>
  __device__ __forceinline__ void operator()(I) const {}
};

// Operand registers of one score tile.  Kept outside score_tile so that the
// phase before it can issue the first kAhead reads early (the K tile is
// already valid then): the first MFMAs of the score phase find their operands
// in registers instead of waiting for LDS.
template <int D, int kAheadMax = FA355_SCORE_AHEAD>
struct ScoreOps {
  static constexpr int kMfmas = 2 * (D / 16);  // MFMA i: slab i / 2, block i % 2
  static constexpr int kAhead = kAheadMax < kMfmas ? kAheadMax : kMfmas;
  static constexpr int kSlots = kAhead + 2;    // a slot is refilled two MFMAs after its use
  u32x4 a[kSlots];
  template <int I>
  __device__ __forceinline__ void issue(uint32_t kaddr) {
    a[I % kSlots] = lds_read128<(I / 2) * Bf16Layout<D>::kKSlab + (I % 2) * 1024>(kaddr);
  }
};

// PRE: the first kAhead reads were issued by the caller (ScoreOps::issue<0..
// kAhead-1>, in order, with no LDS operation of its own after them).
template <int D, typename T = __bf16, bool PRE = false, int kAheadMax = FA355_SCORE_AHEAD, typename Work = NoWork>
__device__ __forceinline__ void score_tile(uint32_t kaddr, const typename Elem<T>::v8 (&qf)[D / 16],
                                           f32x16 (&sacc)[2], ScoreOps<D, kAheadMax>& ops,
                                           Work&& work = Work{}) {
  using V8 = typename Elem<T>::v8;
  using Ops = ScoreOps<D, kAheadMax>;
  constexpr int kMfmas = Ops::kMfmas, kAhead = Ops::kAhead, kSlots = Ops::kSlots;
  static_assert(kMfmas % 2 == 0 && kAhead % 2 == 0, "operands are read two MFMAs at a time");
  if constexpr (!PRE)
    static_for<kAhead>([&](auto ic) { ops.template issue<decltype(ic)::value>(kaddr); });
  sacc[0] = f32x16{};
  sacc[1] = f32x16{};
  // MFMAs in pairs: one wait covers the operands of both.  The read kAhead
  // MFMAs ahead of each MFMA is issued right before it, so that a read (not a
  // VALU instruction) precedes every MFMA and the previous chunk's
  // transcendental results need no wait states in between.
  static_for<kMfmas / 2>([&](auto jc) {
    constexpr int i0 = 2 * decltype(jc)::value;
    static_for<2>([&](auto hc) {
      constexpr int i = i0 + decltype(hc)::value;
      if constexpr (i + kAhead < kMfmas) ops.template issue<i + kAhead>(kaddr);
      if constexpr (i == i0) {
        // outstanding: the reads of MFMAs i0 .. min(i0 + kAhead, kMfmas - 1)
        constexpr int kLast = i0 + kAhead < kMfmas ? i0 + kAhead : kMfmas - 1;
        lds_wait<(kLast - i0 - 1 > 0 ? kLast - i0 - 1 : 0)>();
        pin(ops.a[i0 % kSlots]);
        pin(ops.a[(i0 + 1) % kSlots]);
      }
      sacc[i % 2] =
          Elem<T>::mfma(__builtin_bit_cast(V8, ops.a[i % kSlots]), qf[i / 2], sacc[i % 2]);
      work(std::integral_constant<int, i>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

template <int D, typename T = __bf16, int kAheadMax = FA355_SCORE_AHEAD, typename Work = NoWork>
__device__ __forceinline__ void score_tile(uint32_t kaddr, const typename Elem<T>::v8 (&qf)[D / 16],
                                           f32x16 (&sacc)[2], Work&& work = Work{}) {
  ScoreOps<D, kAheadMax> ops;
  score_tile<D, T, false>(kaddr, qf, sacc, ops, work);
}

// O^T[db] += V^T[32db.., 16-key step] P^T for the four 16-key steps of a tile.
// Lane j of 16-lane group g points at 4 consecutive d of V row key0 + j/4,
// where the group's d0 = 32db + 16(g%2) and key0 = 16s + 8(g/2) [+ 4 for the
// second read]; the transpose hands lane i the column d0 + i.  vaddr = LDS
// address of this lane's piece in slab 0, step 0, first read.
// kExtraFrom: from that MFMA on, the caller's work issues one more LDS read
// after each MFMA (the next score tile's first operands); the waits count them.
template <int D, typename T = __bf16, int kExtraFrom = 1 << 20, typename Work = NoWork>
__device__ __forceinline__ void pv_tile(uint32_t vaddr, const typename Elem<T>::v8 (&pf)[kBN / 16],
                                        f32x16 (&oacc)[D / 32], Work&& work = Work{}) {
  using Lay = Bf16Layout<D>;
  using V8 = typename Elem<T>::v8;
  constexpr int kAheadMax = 4;
  constexpr int kBlocks = D / 32;
  constexpr int kMfmas = (kBN / 16) * kBlocks;  // MFMA i: step i / kBlocks, block i % kBlocks
  constexpr int kAhead = kAheadMax < kMfmas ? kAheadMax : kMfmas;
  constexpr int kSlots = kAhead + 2;            // a slot is refilled two MFMAs after its use
  u32x2 v[kSlots][2];
  auto issue = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    constexpr int s = i / kBlocks, db = i % kBlocks;
    constexpr int off = db * Lay::kVSlab + s * 16 * 64;
    v[i % kSlots][0] = lds_tr16<off>(vaddr);
    v[i % kSlots][1] = lds_tr16<off + 4 * 64>(vaddr);
  };
  static_assert(kMfmas % 2 == 0 && kAhead % 2 == 0, "operands are read two MFMAs at a time");
  static_for<kAhead>(issue);
  // MFMAs in pairs, as in score_tile: one wait covers the operands of both,
  // and the reads kAhead MFMAs ahead of each MFMA are issued right before it.
  // Outstanding at the wait before MFMA i0: the reads of MFMAs i0 ..
  // min(i0 + kAhead, kMfmas - 1), plus the extras issued since the reads of
  // MFMA i0 + 1, which went out right before MFMA i0 + 1 - kAhead (or before
  // MFMA 0): those of the chunks of MFMAs i0 + 1 - kAhead .. i0 - 1 that come
  // from kExtraFrom on (the chunk of MFMA i0 runs after the wait).
  auto extras_before = [](auto ic) constexpr {
    constexpr int i0 = decltype(ic)::value;
    constexpr int lo = (i0 + 1 - kAhead > kExtraFrom ? i0 + 1 - kAhead : kExtraFrom);
    return i0 - lo > 0 ? i0 - lo : 0;
  };
  static_for<kMfmas / 2>([&](auto jc) {
    constexpr int i0 = 2 * decltype(jc)::value;
    static_for<2>([&](auto hc) {
      constexpr int i = i0 + decltype(hc)::value;
      constexpr int s = i / kBlocks, db = i % kBlocks;
      if constexpr (i + kAhead < kMfmas) issue(std::integral_constant<int, i + kAhead>{});
      if constexpr (i == i0) {
        constexpr int kLast = i0 + kAhead < kMfmas ? i0 + kAhead : kMfmas - 1;
        constexpr int kX = extras_before(std::integral_constant<int, i0>{});
        constexpr int kN = 2 * (kLast - i0 - 1 > 0 ? kLast - i0 - 1 : 0) + kX;
        static_assert(kN <= 15, "lgkmcnt holds at most 15");
        lds_wait<kN>();
        pin(v[i0 % kSlots][0]);
        pin(v[i0 % kSlots][1]);
        pin(v[(i0 + 1) % kSlots][0]);
        pin(v[(i0 + 1) % kSlots][1]);
      }
      u32x2(&cur)[2] = v[i % kSlots];
      const u32x4 a = {cur[0][0], cur[0][1], cur[1][0], cur[1][1]};
      oacc[db] = Elem<T>::mfma(__builtin_bit_cast(V8, a), pf[s], oacc[db]);
      work(std::integral_constant<int, i>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// Row statistics combined across the two half-waves (lanes l and l ^ 32 hold
// the two halves of a query column's keys).
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup -> (batch*head, query tile).  MI355X deals consecutive workgroup
// ids round-robin over its 8 XCDs, each with its own L2.  Every XCD gets
// whole heads, so the query tiles of a head share one L2 for their repeated
// reads of that head's K and V.  Causal tiles differ in work (tile i streams
// i+1 blocks of keys): within an XCD the heads are taken two at a time, and
// the tiles of each pair run longest first (longest-processing-time order,
// which keeps the XCD's CUs evenly loaded to the end).  Pairs rather than all
// of the XCD's heads at once keep the K and V being streamed near the size of
// the L2 instead of re-fetching them from beyond it.
template <bool CAUSAL>
__device__ __forceinline__ void map_tile(int bid, int BH, int nq, int& bh, int& qt) {
  constexpr int kXcds = 8;
  if (BH % kXcds == 0) {
    const int hp = BH / kXcds;            // heads per XCD
    const int xcd = bid % kXcds, slot = bid / kXcds;
    if (CAUSAL) {
      const int G = hp % 2 == 0 ? 2 : 1;  // heads per longest-first group
      const int grp = slot / (G * nq), r = slot % (G * nq);
      qt = nq - 1 - r / G;
      bh = xcd * hp + grp * G + r % G;
    } else {
      bh = xcd * hp + slot / nq;
      qt = slot % nq;
    }
  } else if (CAUSAL) {
    qt = nq - 1 - bid / BH;
    bh = bid % BH;
  } else {
    bh = bid / nq;
    qt = bid % nq;
  }
}

// Persistent launches: workgroup b's k-th (batch*head, query tile), or false
// when it has no k-th.  The workgroups of one XCD (ids congruent mod 8) share
// that XCD's heads, as in map_tile.  The XCD's tiles are ranked in groups of
// two heads (one when the XCD holds an odd count), and inside a group level
// by level, causal levels longest first (non-causal: one head at a time, its
// tiles in order); round k hands out ranks k*W .. k*W+W-1
// to the XCD's W workgroups, in reverse order on odd rounds.  Causal tile
// lengths fall linearly with the level, so the reversal pairs a round's long
// tiles with the next round's short ones and every workgroup ends up with
// about the same number of key tiles.
template <bool CAUSAL>
__device__ __forceinline__ bool persist_item(int b, int k, int grid, int BH, int nq, int& bh,
                                             int& qt) {
  constexpr int kXcds = 8;
  int xcd = 0, slot = b, W = grid, hp = BH;
  if (BH % kXcds == 0 && grid % kXcds == 0) {
    xcd = b % kXcds;
    slot = b / kXcds;
    W = grid / kXcds;
    hp = BH / kXcds;
  }
  const int r = k * W + ((k & 1) ? W - 1 - slot : slot);
  if (r >= hp * nq) return false;
  const int G = CAUSAL && hp % 2 == 0 ? 2 : 1;
  const int grp = r / (G * nq), rr = r - grp * (G * nq);
  const int lev = rr / G;
  qt = CAUSAL ? nq - 1 - lev : lev;
  bh = xcd * hp + grp * G + (rr - lev * G);
  return true;
}

// 32-bit LDS read from inline asm (see lds_tr16), for the block-sparse tile list.
__device__ __forceinline__ uint32_t lds_read32(uint32_t lds_addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(lds_addr));
  return v;
}

template <int D, bool CAUSAL, int MODE, typename T = __bf16>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(FA355_BF16_OCCUPANCY, FA355_BF16_OCCUPANCY))) void
fa_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ Lse, int N,
    int BH, int num_qtiles, float scale, float scale_log2, ModeArgs split_args) {
  constexpr bool SPLIT = MODE == kSplit;
  constexpr bool SPARSE = MODE == kSparse;
  // Persistent: the grid holds one workgroup per CU and each walks its list
  // of query tiles (persist_item).  The K/V ring runs on across the tiles:
  // the refills that would reload past the end of one tile's keys fetch the
  // next tile's first K and V tiles instead, so that the next prologue finds
  // them in LDS.  This needs every query tile to stream at least kStages key
  // tiles (N > (kStages - 1) * kBN, which the host checks): a tile's loop
  // loads only the next tile's keys, never the one after it.
  constexpr bool PERSIST = MODE == kPersist;
  static_assert(!PERSIST || kVStages == kStages, "persistent launches keep K and V in step");
  using V8 = typename Elem<T>::v8;  // eight 16-bit elements of type T
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dimension");
  using Lay = Bf16Layout<D>;
  constexpr int kVmPerTile = Lay::kLoadsPerWave;    // direct loads a wave issues per tile
  constexpr int kMf = D / 8;                        // MFMAs per stream per tile (16 at d = 128)
  constexpr bool kLhInPv = false;                   // where the rounded-P sum is taken (lh_step)
  // 16-bit outputs go through the LDS staging area: with a dedicated area
  // always (not the block-sparse path, whose tile list sits past the rings),
  // otherwise in launches that are not persistent (the ring is free at the
  // end).  The split path writes float32 partials directly.
  constexpr bool kStagedStore =
      !SPLIT && (FA355_STAGE_DEDICATED ? !SPARSE : !PERSIST);
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index as a scalar: everything derived from it (row ranges, tile
  // counts, load destinations) stays in scalar registers and branches on it
  // are uniform.
  const int wave = tid >> 6;
  // The same as a scalar, for the load destinations (LDS addresses are set
  // through M0, a scalar register).
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int qi = lane & 31;  // query column of this lane inside the wave's 32
  const int hh = lane >> 5;  // half-wave

  int bh, qt, split = 0;
  if constexpr (PERSIST) {
    if (!persist_item<CAUSAL>(blockIdx.x, 0, gridDim.x, BH, num_qtiles, bh, qt)) return;
  } else if (SPLIT && CAUSAL) {
    // Longest first: query tiles from the last (most visible keys) down, all
    // key ranges of a tile together (they have equal work); heads fastest, so
    // that consecutive workgroups, which land on different XCDs, keep each
    // head on one XCD.
    const int per_level = BH * split_args.num_splits;
    const int level = blockIdx.x / per_level;
    const int r = blockIdx.x - level * per_level;
    split = r / BH;
    bh = r - split * BH;
    qt = num_qtiles - 1 - level;
  } else if (SPLIT) {  // split index fastest, then query tile, then head
    const int q = blockIdx.x / split_args.num_splits;
    split = blockIdx.x - q * split_args.num_splits;
    bh = q / num_qtiles;
    qt = q - bh * num_qtiles;
  } else if (SPARSE && !CAUSAL) {
    // Query tiles outermost, first to last: how much a tile streams depends
    // on the mask, and the first rows are the ones a sparse pattern most
    // often makes global (seeing every key), so they start first.  Heads stay
    // whole on one XCD as in map_tile.
    constexpr int kXcds = 8;
    if (BH % kXcds == 0) {
      const int hp = BH / kXcds, xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
      qt = slot / hp;
      bh = xcd * hp + slot % hp;
    } else {
      qt = blockIdx.x / BH;
      bh = blockIdx.x % BH;
    }
  } else {
    map_tile<CAUSAL>(blockIdx.x, BH, num_qtiles, bh, qt);
  }
  // Per-lane operand offsets (constant over the kernel).
  const int arow = key_of_row(qi);
  const int k_lane = arow * 32 + 16 * (hh ^ ((arow >> 3) & 1));
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_lane = (8 * (g16 >> 1) + (j16 >> 2)) * 64 + 2 * (16 * (g16 & 1) + 4 * (j16 & 3));
  const uint32_t smem_lds = lds_address(smem);
  auto k_addr = [&](int slot) { return smem_lds + Lay::kOffK + slot * Lay::kTileBytes + k_lane; };
  auto v_addr = [&](int slot) { return smem_lds + Lay::kOffV + slot * Lay::kTileBytes + v_lane; };
  uint32_t k_off[kVmPerTile], v_off[kVmPerTile];
#pragma unroll
  for (int r = 0; r < kVmPerTile; ++r) {
    k_off[r] = tile_lane_offset<D, false>(wave, lane, r);
    v_off[r] = tile_lane_offset<D, true>(wave, lane, r);
  }

  // K/V ring slot of the current query tile's first key tile (persistent
  // launches carry the ring position over from tile to tile).
  int ring = 0;
  V8 qf[D / 16];  // Q^T as the B operand of S^T = K Q^T: lane holds d = 16s + 8hh + (0..7)
  auto load_q = [&](int bh_q, int qt_q) {
    const int qr = min(qt_q * kBM + wave * 32 + qi, N - 1);
    const uint16_t* qp = Q + (size_t)bh_q * N * D + (size_t)qr * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(qp + 16 * s));
  };
  load_q(bh, qt);
  for (int nth = 0;; ++nth) {
    bool has_next = false;  // persistent: this workgroup has a next query tile (nbh, nqt)
    int nbh = 0, nqt = 0;
    if constexpr (PERSIST)
      has_next = persist_item<CAUSAL>(blockIdx.x, nth + 1, gridDim.x, BH, num_qtiles, nbh, nqt);
    const int q0 = qt * kBM;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* Kb = K + head;
    const uint16_t* Vb = V + head;

    const int wq0 = q0 + wave * 32;  // first query row of this wave
    const int qrow = wq0 + qi;

    // Keys of this workgroup: [kv_lo, kv_hi) (the whole row without SPLIT).
    // Tiles the workgroup streams, and the prefix of them this wave needs.
    static_assert(kSplitRows % kBM == 0 && kBN == kSplitKeys, "split blocks hold whole tiles");
    int kv_lo = 0, kv_hi = N;
    if (SPLIT) split_range(split, split_args.num_splits, q0 / kSplitRows, N, CAUSAL, kv_lo, kv_hi);
    const int kv_end = CAUSAL ? min(kv_hi, q0 + kBM) : kv_hi;
    int n_tiles = kv_end > kv_lo ? (kv_end - kv_lo + kBN - 1) / kBN : 0;
    int my_tiles = 0;
    if (wq0 < N) {
      const int wave_end = CAUSAL ? min(kv_hi, wq0 + 32) : kv_hi;
      my_tiles = wave_end > kv_lo ? (wave_end - kv_lo + kBN - 1) / kBN : 0;
    }

    // Block-sparse: the tile list, built in LDS past the K and V rings.  It
    // holds, in increasing order, the key blocks that at least one of this
    // workgroup's 64-row query blocks may see, each as (key block | bits << 24)
    // with bit r set when query block r of the workgroup sees it.
    const uint32_t list_off = Lay::kBytes;
    if constexpr (SPARSE) {
      constexpr int kQBlocks = kBM / kMaskBlock;
      static_assert(kBN == kMaskBlock && kBM % kMaskBlock == 0, "mask blocks are tiles");
      uint32_t* list = reinterpret_cast<uint32_t*>(smem + list_off);
      const int nb = (N + kMaskBlock - 1) / kMaskBlock;
      int* counts = reinterpret_cast<int*>(list + nb);
      const int qb0 = q0 / kMaskBlock;
      const int kb_end = CAUSAL ? min(nb, qb0 + kQBlocks) : nb;
      const int qblocks = min(kQBlocks, nb - qb0);
      const uint8_t* mrow =
          split_args.mask + ((size_t)mask_head(split_args, bh) * nb + qb0) * (size_t)nb;
      int total = 0;
      for (int c = 0; c < kb_end; c += kThreads) {
        const int kb = c + tid;
        uint32_t bits = 0;
        if (kb < kb_end) {
          for (int r = 0; r < qblocks; ++r)
            if ((!CAUSAL || kb <= qb0 + r) && mrow[(size_t)r * nb + kb] != 0) bits |= 1u << r;
        }
        const uint64_t bal = __builtin_amdgcn_ballot_w64(bits != 0);
        if (lane == 0) counts[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int before = total, all = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const int cw = counts[w];
          before += w < wave ? cw : 0;
          all += cw;
        }
        if (bits != 0)
          list[before + __builtin_popcountll(bal & ((1ull << lane) - 1))] =
              (uint32_t)kb | (bits << 24);
        total += all;
        __syncthreads();
      }
      n_tiles = total;
      my_tiles = wq0 < N ? total : 0;
    }
    const int last = n_tiles - 1;
    // Leading tiles of the range that every row of the workgroup sees whole:
    // inside N and, under the causal mask, before the workgroup's first row.
    int n_safe = 0;
    if constexpr (!SPARSE) {
      int safe_end = min(kv_end, N & ~(kBN - 1));
      if (CAUSAL) safe_end = min(safe_end, q0);
      n_safe = safe_end > kv_lo ? (safe_end - kv_lo) / kBN : 0;
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
    float l_run = 0.f;   // this half-wave's part of the denominator (float32 P)
    float lh_run = 0.f;  // the same sum over P as rounded for the P V MFMAs

    const __amdgpu_buffer_rsrc_t k_rsrc = head_resource(Kb, N * D * 2);
    const __amdgpu_buffer_rsrc_t v_rsrc = head_resource(Vb, N * D * 2);
    const size_t next_head = (size_t)nbh * N * D;
    const __amdgpu_buffer_rsrc_t k_rsrc_next = head_resource(K + next_head, N * D * 2);
    const __amdgpu_buffer_rsrc_t v_rsrc_next = head_resource(V + next_head, N * D * 2);
    constexpr uint32_t kNextTile = 1u << 31;  // entry flag: a key tile of the next query tile
    // Tile t of the workgroup as an entry: its key block, plus (block-sparse
    // path) which query blocks see it.  Dense and split paths: key block
    // kv_lo / kBN + t; block-sparse: the t-th list entry, read from LDS with
    // asm (callers wait with lds_wait<0> and pin the result).  Entries past the
    // last tile repeat it (the ring's final refills reload the last tile), or,
    // persistent with a next query tile, stand for that tile's key tiles.
    auto entry = [&](int tile) -> uint32_t {
      if constexpr (PERSIST) {
        if (has_next && tile > last) return (uint32_t)(tile - n_tiles) | kNextTile;
      }
      const int t = min(tile, last);
      if constexpr (SPARSE) return lds_read32(smem_lds + list_off + 4 * t);
      else return (uint32_t)(kv_lo / kBN + t);
    };
    // Orders uses of an entry after the lds_wait, and moves it to a scalar
    // register (it is the same in every lane).
    auto pin_entry = [](uint32_t& e) {
      asm volatile("" : "+v"(e));
      e = __builtin_amdgcn_readfirstlane(e);
    };
    auto entry_kv0 = [](uint32_t e) {
      return (int)(SPARSE ? e & 0xFFFFFFu : PERSIST ? e & ~kNextTile : e) * kBN;
    };
    // Does this wave's 64-row query block see the tile at all?
    auto entry_seen = [&](uint32_t e) { return !SPARSE || ((e >> (24 + (wave >> 1))) & 1u) != 0; };
    auto load_k = [&](int slot, uint32_t e) {
      load_tile_direct<D>(smem, Lay::kOffK + slot * Lay::kTileBytes,
                          PERSIST && (e & kNextTile) ? k_rsrc_next : k_rsrc, entry_kv0(e), wave_s,
                          k_off);
    };
    auto load_v = [&](int slot, uint32_t e) {
      load_tile_direct<D>(smem, Lay::kOffV + slot * Lay::kTileBytes,
                          PERSIST && (e & kNextTile) ? v_rsrc_next : v_rsrc, entry_kv0(e), wave_s,
                          v_off);
    };

    // The same for a key tile of this query tile's own range (no flag to test).
    auto load_k_own = [&](int slot, uint32_t tile) {
      load_tile_direct<D>(smem, Lay::kOffK + slot * Lay::kTileBytes, k_rsrc, (int)tile * kBN,
                          wave_s, k_off);
    };
    auto load_v_own = [&](int slot, uint32_t tile) {
      load_tile_direct<D>(smem, Lay::kOffV + slot * Lay::kTileBytes, v_rsrc, (int)tile * kBN,
                          wave_s, v_off);
    };

    // Softmax of one tile's raw scores s, in two halves.  Stage 1: mask, row
    // maximum, reference update, the exponentials of block 0 and their sum.
    // Stage 2: the exponentials of block 1, the row sum into l_run, and P^T as
    // bf16 B operands of O^T += V^T P^T (16-key step s2 takes elements
    // 8(s2%2) .. 8(s2%2)+7 of block s2/2, i.e. keys 16 s2 + 8hh + (0..7)).
    // s element 4g+r of block kb is key kv0 + 32kb + key_of_row(8g + 4hh + r).
    // Returns whether the tile needed a mask for this wave (uniform).
    auto mask_tile = [&](uint32_t ent, f32x16(&sc)[2]) -> bool {
      const int kv0 = entry_kv0(ent);
      const bool hidden = !entry_seen(ent);  // a key block this wave's query block does not see
      const bool need_mask = hidden || (kv0 + kBN > N) || (CAUSAL && kv0 + kBN - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kv0 + 32 * kb + key_of_row(8 * (e >> 2) + 4 * hh + (e & 3));
            if (hidden || key >= N || (CAUSAL && key > qrow)) sc[kb][e] = kNegInf;
          }
      }
      return need_mask;
    };
    // The softmax of a tile as numbered steps, so that each MFMA of a phase can
    // be given its share (step s of NS goes after MFMA s * kMf / NS).
    // Stage 1 (18 steps): the row maximum as a chain of three-input maxima
    // (two per step), the half-wave exchange and reference update, eight pairs
    // of exponentials of block 0, their sum.
    // Stage 2 (17 steps): eight pairs of exponentials of block 1, the row sum
    // into l_run, eight pairs of bf16 conversions into the P^T operands (whose
    // rounded values are summed into lh_run: right after each conversion at
    // d >= 128, under that tile's P V MFMAs at d <= 64, lh_step below).  L
    // takes the sum of the float32 probabilities (l_run):
    // the sum of their bf16 roundings would move L by up to 2^-8 on rows with
    // few keys.  O is divided by the sum of the rounded values (lh_run), the
    // weights the P V MFMAs actually applied, so that O is their convex
    // combination of V rows: divided by l_run instead, a row dominated by one
    // key carries that key's rounding error (up to 2^-8 |v|) into O on top of
    // O's own bf16 rounding, which exceeded 2e-2 on rows with |O| near 4 under
    // the large-logits workload.
    struct SoftmaxState {
      float m, alpha, half_sum;
      bool need;
    };
    // Factor that moves lh_run to the reference of the tile whose P^T is in
    // the P V operands (that tile's alpha); set with P^T, used when its
    // rounded values are summed during that tile's P V MFMAs.
    float lh_alpha = 1.f;
    constexpr int kStage1Steps = 18, kStage2Steps = 17;
    auto stage1_step = [&](auto sic, f32x16(&sc)[2], SoftmaxState& st) {
      constexpr int sidx = decltype(sic)::value;
      if constexpr (sidx < 8) {
        constexpr int kb = sidx >> 2, e = 4 * (sidx & 3);
        if constexpr (sidx == 0) st.m = fmaxf(sc[0][0], sc[0][1]);
        else st.m = fmaxf(fmaxf(st.m, sc[kb][e]), sc[kb][e + 1]);
        st.m = fmaxf(fmaxf(st.m, sc[kb][e + 2]), sc[kb][e + 3]);
      } else if constexpr (sidx == 8) {
        const float mx = max_halves(st.m);
        const float cand = mx * scale_log2;  // -inf for a fully masked tile
        st.need = cand > base_run + kTau;
        const float base_new = st.need ? cand : base_run;
        st.alpha = fast_exp2(base_run - base_new);
        m_ref = st.need ? mx : m_ref;
        base_run = base_new;
      } else if constexpr (sidx < 17) {
        constexpr int e = 2 * (sidx - 9);
        sc[0][e] = fast_exp2(__builtin_fmaf(sc[0][e], scale_log2, -base_run));
        sc[0][e + 1] = fast_exp2(__builtin_fmaf(sc[0][e + 1], scale_log2, -base_run));
      } else {
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = sc[0][2 * i] + sc[0][2 * i + 1];
        st.half_sum = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
      }
    };
    auto stage2_step = [&](auto sic, f32x16(&sc)[2], SoftmaxState& st, V8(&pfo)[kBN / 16]) {
      constexpr int sidx = decltype(sic)::value;
      if constexpr (sidx < 8) {
        constexpr int e = 2 * sidx;
        sc[1][e] = fast_exp2(__builtin_fmaf(sc[1][e], scale_log2, -base_run));
        sc[1][e + 1] = fast_exp2(__builtin_fmaf(sc[1][e + 1], scale_log2, -base_run));
      } else if constexpr (sidx == 8) {
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = sc[1][2 * i] + sc[1][2 * i + 1];
        const float lsum =
            st.half_sum + (((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7])));
        l_run = __builtin_fmaf(l_run, st.alpha, lsum);
      } else {
        // pair k of the 32 conversions: elements 4k .. 4k+3 of the tile's keys
        constexpr int k = sidx - 9;
        constexpr int s2 = k >> 1, j0 = 4 * (k & 1);
#pragma unroll
        for (int j = j0; j < j0 + 4; ++j) pfo[s2][j] = (T)sc[s2 >> 1][8 * (s2 & 1) + j];
        if constexpr (kLhInPv) {
          if constexpr (k == 7) lh_alpha = st.alpha;
        } else {
          if constexpr (k == 0) lh_run *= st.alpha;
          lh_run = Elem<T>::template add_pair<j0 / 2>(pfo[s2], lh_run);
          lh_run = Elem<T>::template add_pair<j0 / 2 + 1>(pfo[s2], lh_run);
        }
      }
    };
    // The sum of the rounded P^T operands pfo into lh_run, as 8 steps (two
    // pairs each) that run under the P V MFMAs reading those operands; at
    // d = 128 and 256 it is taken right after each conversion instead (kLhInPv
    // false), which measured faster there (d = 64 is VALU-bound and gains from
    // moving the work into the P V phase).
    constexpr int kLhSteps = kLhInPv ? 8 : 0;
    auto lh_step = [&](auto sic, const V8(&pfo)[kBN / 16]) {
      constexpr int k = decltype(sic)::value;
      constexpr int s2 = k >> 1, p0 = 2 * (k & 1);
      if constexpr (k == 0) lh_run *= lh_alpha;
      lh_run = Elem<T>::template add_pair<p0>(pfo[s2], lh_run);
      lh_run = Elem<T>::template add_pair<p0 + 1>(pfo[s2], lh_run);
    };
    // The tile's softmax without its row maximum.  When the previous tile
    // moved no reference point of the wave, the next tile's scores are
    // exponentiated against the current reference right away: the row
    // maximum, its half-wave exchange and the reference update are skipped.
    // The raw scores are kept, and the tile's half-row sums of the
    // probabilities are checked at the end: if one exceeds kFastLimit, the
    // tile is redone along the path with the maximum (which moves the
    // reference), and the wave returns to that path for the next tile.
    // Otherwise every probability of the tile is at most kFastLimit (they
    // are non-negative and their sum is): the reference may lag the row
    // maximum by up to 16 instead of kTau (base 2), which float32 sums and
    // 16-bit P hold with room to spare, and by shift invariance the
    // normalised result is the same softmax.
    constexpr float kFastLimit = 65536.f;  // 2^16
    struct FastState {
      float l, lh;   // this tile's sums of the float32 and of the rounded probabilities
      float tp[8][2];  // probabilities of pair k until their P^T step is free
    };
    // Pair k (0..15) of the tile: elements 2(k%8), 2(k%8)+1 of block k/8,
    // i.e. elements j, j+1 (j = 2(k%4)) of P^T step k/4.  Phase 1 takes
    // pairs 0..7 (steps 0, 1) under the P V MFMAs: the exponentials of pair
    // k after MFMA k*kMf/8, its conversion once MFMA (k/4 + 1)*kBlocks - 1,
    // the last to read the old step, has gone (kBlocks = D/32 MFMAs per
    // step); phase 3 takes pairs 8..15 (steps 2, 3, free by then).
    constexpr int kPvBlocks = D / 32;
    auto fast_step = [&](auto ic, auto phase3_c, f32x16(&sc)[2], FastState& fs,
                         V8(&pfo)[kBN / 16]) {
      constexpr int c = decltype(ic)::value;
      constexpr bool P3 = decltype(phase3_c)::value;
      static_for<8>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;        // pair within the phase
        constexpr int k = kk + (P3 ? 8 : 0);            // pair of the tile
        constexpr int kb = k / 8, e = 2 * (k % 8);      // block and element
        constexpr int s2 = k / 4, j = 2 * (k % 4);      // P^T step and element
        constexpr int ce = kk * kMf / 8;                // chunk of the exponentials
        constexpr int free_at = P3 ? 0 : (s2 + 1) * kPvBlocks - 1;
        constexpr int cc0 = kMf >= 16 ? ce + 1 : ce;
        constexpr int cc = cc0 > free_at ? cc0 : free_at;  // chunk of sum and conversion
        if constexpr (c == ce) {
          fs.tp[kk][0] = fast_exp2(__builtin_fmaf(sc[kb][e], scale_log2, -base_run));
          fs.tp[kk][1] = fast_exp2(__builtin_fmaf(sc[kb][e + 1], scale_log2, -base_run));
        }
        if constexpr (c == cc) {
          fs.l = (k == 0 ? fs.tp[kk][0] : fs.l + fs.tp[kk][0]) + fs.tp[kk][1];
          pfo[s2][j] = (T)fs.tp[kk][0];
          pfo[s2][j + 1] = (T)fs.tp[kk][1];
          fs.lh = Elem<T>::template add_pair<j / 2>(pfo[s2], k == 0 ? 0.f : fs.lh);
        }
      });
    };
    // The tile again along the reference rule, for a wave whose check
    // failed: row maximum, reference update, the output and both sums moved
    // to the new reference, then every probability from the raw scores.  The
    // arithmetic of each step is that of stages 1 and 2.
    // Returns the factor that moves the output to the new reference point
    // (1 when no row of the wave moved); the caller applies it.
    auto redo_tile = [&](const f32x16(&sc)[2], V8(&pfo)[kBN / 16], bool& moved) -> float {
      float m = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = (kb == 0 ? 2 : 0); e < 16; e += 2) m = fmaxf(fmaxf(m, sc[kb][e]), sc[kb][e + 1]);
      const float mx = max_halves(m);
      const float cand = mx * scale_log2;
      const bool need = cand > base_run + kTau;
      const float base_new = need ? cand : base_run;
      const float alpha = fast_exp2(base_run - base_new);
      m_ref = need ? mx : m_ref;
      base_run = base_new;
      moved = __builtin_amdgcn_ballot_w64(need) != 0;
      float lsum = 0.f, lhs = lh_run * alpha;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int kb = k / 8, e = 2 * (k % 8), s2 = k / 4, j = 2 * (k % 4);
        const float p0 = fast_exp2(__builtin_fmaf(sc[kb][e], scale_log2, -base_run));
        const float p1 = fast_exp2(__builtin_fmaf(sc[kb][e + 1], scale_log2, -base_run));
        lsum += p0 + p1;
        pfo[s2][j] = (T)p0;
        pfo[s2][j + 1] = (T)p1;
        lhs = Elem<T>::add_pair_rt(pfo[s2], j / 2, lhs);
        // one pair at a time: all exponentials at once would need 32 more
        // registers at a point where both score tiles are live
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run = __builtin_fmaf(l_run, alpha, lsum);
      lh_run = lhs;
      return alpha;
    };
    // Steps of a stage that belong after MFMA i of a kMf-MFMA phase.
    auto run_steps = [&](auto ic, auto nsteps_ic, auto&& step) {
      constexpr int i = decltype(ic)::value;
      constexpr int NS = decltype(nsteps_ic)::value;
      static_for<NS>([&](auto sic) {
        constexpr int sidx = decltype(sic)::value;
        if constexpr (sidx * kMf / NS == i) step(sic);
      });
    };
    auto stage1 = [&](f32x16(&sc)[2], SoftmaxState& st) {
      static_for<kStage1Steps>([&](auto sic) { stage1_step(sic, sc, st); });
    };
    auto stage2 = [&](f32x16(&sc)[2], SoftmaxState& st, V8(&pfo)[kBN / 16]) {
      static_for<kStage2Steps>([&](auto sic) { stage2_step(sic, sc, st, pfo); });
    };
    // Empty asm that ties values to this point of the program: the compiler
    // would otherwise sink them past the next branch, next to their use.
    auto pin_scores = [&](f32x16(&sc)[2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x4 w = {__float_as_uint(sc[kb][4 * q]), __float_as_uint(sc[kb][4 * q + 1]),
                     __float_as_uint(sc[kb][4 * q + 2]), __float_as_uint(sc[kb][4 * q + 3])};
          pin(w);
          sc[kb][4 * q] = __uint_as_float(w[0]);
          sc[kb][4 * q + 1] = __uint_as_float(w[1]);
          sc[kb][4 * q + 2] = __uint_as_float(w[2]);
          sc[kb][4 * q + 3] = __uint_as_float(w[3]);
        }
    };
    auto pin_probs = [&](V8(&pfo)[kBN / 16]) {
#pragma unroll
      for (int s2 = 0; s2 < kBN / 16; ++s2) {
        u32x4 w = __builtin_bit_cast(u32x4, pfo[s2]);
        pin(w);
        pfo[s2] = __builtin_bit_cast(V8, w);
      }
      asm volatile("" : "+v"(l_run), "+v"(lh_run));
    };

    // A workgroup whose key range is empty (a split past the causal diagonal)
    // skips straight to the epilogue, which then writes L = -inf and O = 0.
    // Persistent tiles always stream keys.
    if (PERSIST || n_tiles > 0) {
      // Prologue.  Ring slots: K tile j lives in slot j % kStages, V tile j in
      // slot j % kVStages.  Iteration t reads V_t and K_{t+2}.  It refills the
      // slot of K_{t+1} (read in iteration t-1) with K_{t+1+kStages}, and the
      // V slot freed by iteration t-1 with V_{t-1+kVStages}.  Before iteration
      // 0, K_0..K_2 and V_0 must have landed.  With equal ring depths S, the
      // loads of the "iterations" 2-S .. -1 are issued here in loop order so
      // that the vmcnt at the end of every iteration stays exact.  K_S goes to
      // the slot of K_0, which the prologue's scores read, so it waits for the
      // second barrier.
      //
      // Persistent launches: tile j of the current query tile is in slot
      // (ring + j) % kStages, and the tails of the previous query tile's loop
      // have already loaded (and waited for) this prologue's tiles.
      auto wrap = [](int x) { return x >= kStages ? x - kStages : x; };
      uint32_t e0 = entry(0);
      if (!PERSIST || nth == 0) {
        uint32_t e1 = entry(1), e2 = entry(2);
        if constexpr (SPARSE) {
          lds_wait<0>();
          pin_entry(e0);
          pin_entry(e1);
          pin_entry(e2);
        }
        load_k(0, e0);
        load_k(1, e1);
        load_k(2, e2);
        load_v(0, e0);
        if constexpr (kVStages == kStages) {
#pragma unroll
          for (int j = 3; j < kStages; ++j) {
            uint32_t ej = entry(j), ev = entry(j - 2);
            if constexpr (SPARSE) {
              lds_wait<0>();
              pin_entry(ej);
              pin_entry(ev);
            }
            load_k(j, ej);
            load_v(j - 2, ev);
          }
          uint32_t ev = entry(kStages - 2);
          if constexpr (SPARSE) {
            lds_wait<0>();
            pin_entry(ev);
          }
          load_v(kStages - 2, ev);
          wait_vmcnt<(2 * (kStages - 3) + 1) * kVmPerTile>();  // K_0..K_2 and V_0 have landed
        } else {
          wait_vmcnt<0>();  // a 2-deep V ring: iteration 0 loads V_1
        }
        block_sync();
      }

      f32x16 sA[2], sB[2];  // raw scores / probabilities of two consecutive tiles
      V8 pf[kBN / 16];  // P^T of the tile whose P V is next
      // Q has landed here on every path, also in waves with no rows (which
      // never read it): otherwise the compiler keeps the load pending and
      // waits for every load in flight before the next Q load reuses qf.
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        u32x4 w = __builtin_bit_cast(u32x4, qf[s]);
        pin(w);
        qf[s] = __builtin_bit_cast(V8, w);
      }
      // The next plain tile may skip its row maximum (see FastState).
      bool fast = false;
      if (my_tiles > 0) {
        score_tile<D, T>(k_addr(ring), qf, sA);
        score_tile<D, T>(k_addr(wrap(ring + 1)), qf, sB);
        mask_tile(e0, sA);
        SoftmaxState st;
        stage1(sA, st);
        stage2(sA, st, pf);
        fast = __builtin_amdgcn_ballot_w64(st.need) == 0;
      }
      uint32_t es = entry(kStages);
      if constexpr (SPARSE) {
        lds_wait<0>();
        pin_entry(es);
      }
      block_sync();  // every wave is done reading K_0 before its slot is refilled
      load_k(ring, es);

      // One tile.  On entry pf holds P_t and cur the raw scores of tile t+1;
      // nxt receives tile t+2.  sk = t % kStages is the K ring position (K_{t+2}
      // is in slot (sk+2) % kStages); svs = t % kVStages is V_t's slot.
      // The loads of later tiles are issued between the P V MFMAs (the V load
      // after the third, the K load half way) rather than all at the top:
      // eight waves issuing them at once right after the barrier queue up in
      // the address unit.  Issued there, their LDS writes tend to land during
      // the score phase, whose b128 operand reads leave LDS bandwidth to spare,
      // rather than during the P V phase, whose transposing reads need about
      // all of it (V issued in the score phase measured 0.4-1% slower).  With
      // a 2-deep V ring the V load goes first, so that it has the whole
      // iteration to land.
      constexpr bool kShortV = kVStages == 2;
      auto refill_v = [&](auto checked_c, int sk, int svs, uint32_t ev) {
        const int slot = kShortV ? svs ^ 1 : wrap(sk + kStages - 1);
        if constexpr (decltype(checked_c)::value) load_v(slot, ev);
        else load_v_own(slot, ev);
      };
      auto refill_k = [&](auto checked_c, int sk, uint32_t ek) {
        if constexpr (decltype(checked_c)::value) load_k(wrap(sk + 1), ek);
        else load_k_own(wrap(sk + 1), ek);
      };
      // CHECKED false: an iteration whose tiles need no checks, i.e. tile t+1
      // is seen whole by every row of the workgroup (no mask, every wave
      // has it) and the refills name tiles of this query tile's own range.
      auto iteration = [&](auto checked_c, int t, int sk, int svs, f32x16(&cur)[2],
                           f32x16(&nxt)[2]) {
        constexpr bool CHECKED = decltype(checked_c)::value;
        // Entries of this iteration: tile t+1 (masked now), the K tile
        // t+1+kStages and the V tile (t+1 or t-1+kStages) loaded now.  On the
        // block-sparse path they are read here, before any operand read of the
        // iteration is in flight.
        const bool boundary = CHECKED && PERSIST && has_next && t == last;
        uint32_t e_next, e_k, e_v;
        if constexpr (CHECKED) {
          e_next = entry(t + 1);
          e_k = entry(t + 1 + kStages);
          e_v = kShortV ? e_next : entry(t - 1 + kStages);
          if constexpr (SPARSE) {
            lds_wait<0>();
            pin_entry(e_next);
            pin_entry(e_k);
            pin_entry(e_v);
          }
        } else {
          const uint32_t e_t = (uint32_t)(kv_lo / kBN + t);
          e_next = e_t + 1;
          e_k = e_t + 1 + kStages;
          e_v = kShortV ? e_next : e_t - 1 + kStages;
        }
        if (!CHECKED || t + 1 < my_tiles) {
          // The softmax without maximum needs an unmasked tile (decided per
          // wave, from its own rows, so that every launch shape and path
          // takes the same decisions for a row and the results agree bitwise).
          bool fast_now = fast;
          if constexpr (CHECKED) {
            const bool masked = mask_tile(e_next, cur);  // always applied
            fast_now = fast && !masked;
          }
          // The last MFMAs of phase 1 issue the first operand reads of the
          // score phase (K_{t+2} has been valid since the last barrier).
          ScoreOps<D> sops;
          const uint32_t k_next = k_addr(wrap(sk + 2));
          constexpr int kPre = kXPhase ? ScoreOps<D>::kAhead : 0;
          // Loads of later tiles (V early, K half way) and those score-phase
          // reads, issued between the P V MFMAs.
          auto pv_extras = [&](auto ic) {
            constexpr int c = decltype(ic)::value;
            if constexpr (kShortV && c == 0) refill_v(checked_c, sk, svs, e_v);
            if constexpr (!kShortV && c == 2) refill_v(checked_c, sk, svs, e_v);
            if constexpr (c == kMf / 2) refill_k(checked_c, sk, e_k);
            if constexpr (kPre > 0 && c >= kMf - kPre)
              sops.template issue<c - (kMf - kPre)>(k_next);
          };
          if (fast_now) {
            // Phase 1: P V of tile t under the first half of tile t+1's
            // softmax without maximum; phase 3: scores of tile t+2 under the
            // second half.  Then the check.
            FastState fs;
            pv_tile<D, T, kMf - kPre>(v_addr(svs), pf, oacc, [&](auto ic) {
              fast_step(ic, std::false_type{}, cur, fs, pf);
              pv_extras(ic);
            });
            score_tile<D, T, kXPhase>(k_next, qf, nxt, sops, [&](auto ic) {
              fast_step(ic, std::true_type{}, cur, fs, pf);
            });
            bool moved = false;
            float alpha = 1.f;
            if (__builtin_amdgcn_ballot_w64(fs.l > kFastLimit) != 0) {
              // Some probability is too large: the tile again, with the
              // maximum (the raw scores are intact).
              alpha = redo_tile(cur, pf, moved);
              fast = false;
            } else {
              l_run += fs.l;
              lh_run += fs.lh;
            }
            pin_probs(pf);
            // the output moved to the new reference point (rare)
            if (moved) {
#pragma unroll
              for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
            }
          } else {
            // Phase 1: P V of tile t (MFMA) under stage 1 of tile t+1 (VALU).
            SoftmaxState st;
            pv_tile<D, T, kMf - kPre>(v_addr(svs), pf, oacc, [&](auto ic) {
              run_steps(ic, std::integral_constant<int, kStage1Steps>{},
                        [&](auto sic) { stage1_step(sic, cur, st); });
              run_steps(ic, std::integral_constant<int, kLhSteps>{},
                        [&](auto sic) { lh_step(sic, pf); });
              pv_extras(ic);
            });
            pin_scores(cur);
            asm volatile("" : "+v"(st.half_sum), "+v"(st.alpha));

            // Phase 2: move the output to the new reference (rare).
            const bool moved = __builtin_amdgcn_ballot_w64(st.need) != 0;
            if (moved) {
#pragma unroll
              for (int i = 0; i < D / 32; ++i) oacc[i] *= st.alpha;
            }
            fast = !moved;

            // Phase 3: scores of tile t+2 (MFMA) under stage 2 of tile t+1 (VALU).
            score_tile<D, T, kXPhase>(k_next, qf, nxt, sops, [&](auto ic) {
              run_steps(ic, std::integral_constant<int, kStage2Steps>{},
                        [&](auto sic) { stage2_step(sic, cur, st, pf); });
            });
            pin_probs(pf);
          }
        } else {
          if constexpr (kShortV) refill_v(checked_c, sk, svs, e_v);
          // Persistent, last tile with a next query tile: K_{t+1+S} is that
          // tile's K_S, and its slot still holds the next tile's K_0, unread.
          // The next prologue issues it after its first scores, as every
          // prologue does.
          if (!(PERSIST && boundary)) refill_k(checked_c, sk, e_k);
          if (t < my_tiles) {
            pv_tile<D, T>(v_addr(svs), pf, oacc);
            static_for<kLhSteps>([&](auto sic) { lh_step(sic, pf); });
          }
          if constexpr (!kShortV) refill_v(checked_c, sk, svs, e_v);
        }

        // K_{t+3} and V_{t+1} must have landed for every wave before anyone
        // reads them.  Equal rings: both were issued in iteration t+2-S, and the
        // loads of the S-2 later iterations may stay in flight.  2-deep V ring:
        // V_{t+1} was this iteration's first load; only its K load may stay.
        // At a persistent boundary this iteration issued only its V load.
        if constexpr (kShortV) wait_vmcnt<kVmPerTile>();
        else if (PERSIST && boundary) wait_vmcnt<(2 * (kStages - 3) + 1) * kVmPerTile>();
        else wait_vmcnt<2 * (kStages - 2) * kVmPerTile>();
        block_sync();
      };

      // Two tiles per trip so that the two score buffers swap roles instead of
      // being copied (and, with a 2-deep V ring, V slots are constants).
      // Iterations t < t_plain need no checks: tile t+1 is among the n_safe
      // leading tiles that every row of the workgroup sees whole, and the
      // refill K_{t+1+kStages} is still a tile of this range.
      constexpr std::false_type kPlain{};
      constexpr std::true_type kChecked{};
      const int t_plain = max(0, min(n_safe - 1, last - kStages));
      int t = 0, sk = ring;
      for (; t + 1 < t_plain; t += 2) {
        iteration(kPlain, t, sk, kShortV ? 0 : sk, sB, sA);
        iteration(kPlain, t + 1, wrap(sk + 1), kShortV ? 1 : wrap(sk + 1), sA, sB);
        sk = wrap(sk + 2);
      }
      for (; t + 1 < n_tiles; t += 2) {
        iteration(kChecked, t, sk, kShortV ? 0 : sk, sB, sA);
        iteration(kChecked, t + 1, wrap(sk + 1), kShortV ? 1 : wrap(sk + 1), sA, sB);
        sk = wrap(sk + 2);
      }
      if (t < n_tiles) iteration(kChecked, t, sk, kShortV ? 0 : sk, sB, sA);
      // The ring's last refills (clamped repeats of the last tile) are still in
      // flight; let them land before the workgroup can end and its LDS be reused.
      // Persistent with a next query tile: they are that tile's first loads.
      if (!has_next) wait_vmcnt<0>();
    }
    // Persistent: the next query tile's Q, issued before this tile's stores so
    // that waiting for it does not wait for them.
    if (PERSIST && has_next) load_q(nbh, nqt);

    // Epilogue: O^T element 4g+r of block db is O[qrow][32db + 8g + 4hh + r].
    const float l_tot = sum_halves(l_run);
    const float inv = l_tot > 0.f ? 1.f / sum_halves(lh_run) : 0.f;
    // l_tot = sum_j exp2(s_j c - base_run) with base_run = m_ref c - r, where r
    // (exact, from one FMA) is the rounding residual of base_run; hence
    // ln sum_j exp(scale s_j) = m_ref scale + ln l_tot - r ln 2.
    const float resid = __builtin_fmaf(m_ref, scale_log2, -base_run);
    const float lse =
        l_tot > 0.f ? __builtin_fmaf(m_ref, scale, logf(l_tot) - resid * kLn2) : kNegInf;
    if (qrow < N) {
      if (SPLIT) {
        const size_t prow = ((size_t)split * BH + bh) * N + qrow;
        float* orow = split_args.opart + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 o4;
#pragma unroll
            for (int r = 0; r < 4; ++r) o4[r] = oacc[db][4 * g + r] * inv;
            *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * hh) = o4;
          }
        if (hh == 0) split_args.lpart[prow] = lse;
      } else if constexpr (!kStagedStore) {
        uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            T o4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o4[r] = (T)(oacc[db][4 * g + r] * inv);
            *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * hh) =
                __builtin_bit_cast(u32x2, o4);
          }
      }
      if (!SPLIT && hh == 0) Lse[(size_t)bh * N + qrow] = lse;
    }
    if constexpr (kStagedStore) {
      // O through the wave's LDS staging area: the lane of query column qi
      // writes its 8-byte pieces of row qi, then every lane reads 16
      // consecutive bytes of a row and the wave stores 1 KB of consecutive
      // rows per instruction.  The area is this wave's alone, and LDS
      // operations of one wave complete in order.  The swizzle moves a row's
      // 16-byte chunk c to c ^ (row & kSwz); it only changes address bits
      // 4..8, above which the row and the wave's area start (the dynamic LDS
      // of this kernel starts at address 0), so every address is one lane
      // base XOR a constant.  The bases are pinned here: computed once
      // outside the persistent loop, the 24 addresses would be held in
      // registers across it.
      using Lay2 = Bf16Layout<D>;
      constexpr int kRowB = Lay2::kStageRow, kChunks = kRowB / 16;
      constexpr int kSwz = (kChunks < 16 ? kChunks : 16) - 1;
      constexpr int kRowsPerRead = 1024 / kRowB;  // rows per 1 KB read
      static_assert(kRowB % 64 == 0 && Lay2::kStageWave % 2048 == 0 &&
                        Lay2::kStageOff % 2048 == 0, "staging address bits");
      if constexpr (!FA355_STAGE_DEDICATED) {
        // the ring memory: every wave's loads have landed (the loop's end
        // waited for them) once all waves are here
        block_sync();
      }
      // The lane index recomputed here (mbcnt, in a volatile asm that the
      // compiler cannot hoist), so that nothing derived from it is held in
      // registers across the loop.
      int ll;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ll));
      const int lq = ll & 31, lh = ll >> 5;
      const uint32_t wave_area = smem_lds + Lay2::kStageOff + wave_s * Lay2::kStageWave;
      const uint32_t wbase = wave_area + lq * kRowB + ((lq & kSwz) << 4) + 8 * lh;
      const int r0 = ll * 16 / kRowB, c0 = ll * 16 % kRowB / 16;
      const uint32_t rbase = wave_area + r0 * kRowB + ((c0 ^ (r0 & kSwz)) << 4);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          T o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = (T)(oacc[db][4 * g + r] * inv);
          const int chunk = 4 * db + g;  // 16-byte chunk of d = 32db + 8g .. +7
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
              (uintptr_t)(wbase ^ (uint32_t)(chunk << 4))) = __builtin_bit_cast(u32x2, o4);
        }
      // All reads first, then the stores, through a resource spanning this
      // head's N rows: the range check drops the rows past N.
      constexpr int kReads = 32 * kRowB / 1024;
      u32x4 rows_out[kReads];
#pragma unroll
      for (int i = 0; i < kReads; ++i) {
        const uint32_t a = (rbase ^ (uint32_t)(((i * kRowsPerRead) & kSwz) << 4)) + i * 1024;
        rows_out[i] =
            *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)a);
      }
      const __amdgpu_buffer_rsrc_t o_rsrc = head_resource(O + head, N * D * 2);
#pragma unroll
      for (int i = 0; i < kReads; ++i) {
        const uint32_t off = (uint32_t)(wq0 + i * kRowsPerRead + r0) * (uint32_t)kRowB + c0 * 16;
        __builtin_amdgcn_raw_buffer_store_b128(rows_out[i], o_rsrc, off, 0, 0);
      }
    }
    if (!PERSIST || !has_next) break;
    ring = (ring + n_tiles) % kStages;
    bh = nbh;
    qt = nqt;
  }
}

}  // namespace FA355_NS
