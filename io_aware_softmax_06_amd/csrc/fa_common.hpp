// Shared device helpers for the attention forward kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// The kernels' namespace.  A translation unit that builds the kernels with a
// different workgroup configuration (the d = 256 instances) names another
// one, so that the two configurations never share a symbol.
#ifndef FA355_NS
#define FA355_NS fa355
#endif

namespace FA355_NS {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The two 16-bit element types of the MFMA paths.  bf16 and fp16 share every
// layout (2 bytes per element); they differ only in the MFMA instruction and
// in the rounding of P (and of the outputs) to the element type.
template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  using v8 = bf16x8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // acc + x[2i] + x[2i+1] in float32 (v_dot2c_f32_bf16 against (1, 1)).
  template <int I>
  static __device__ __forceinline__ float add_pair(v8 x, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 pair = {x[2 * I], x[2 * I + 1]};
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(pair, one, acc, false);
  }
  // The same with the pair index i (0..3) given at run time (unrolled loops).
  static __device__ __forceinline__ float add_pair_rt(v8 x, int i, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 pair = {x[2 * i], x[2 * i + 1]};
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(pair, one, acc, false);
  }
};
template <>
struct Elem<_Float16> {
  using v8 = f16x8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // acc + x[2i] + x[2i+1] in float32 (v_dot2c_f32_f16 against (1, 1)).
  template <int I>
  static __device__ __forceinline__ float add_pair(v8 x, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 pair = {x[2 * I], x[2 * I + 1]};
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(pair, one, acc, false);
  }
  static __device__ __forceinline__ float add_pair_rt(v8 x, int i, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 pair = {x[2 * i], x[2 * i + 1]};
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(pair, one, acc, false);
  }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// Value held by lane (l ^ 32), the same MFMA column in the other half-wave.
__device__ __forceinline__ float other_half(float v) {
  return __shfl_xor(v, 32, 64);
}

// Key-range split of the forward pass.  The query rows are grouped in blocks
// of kSplitRows; the keys visible to block rb (all N, or with the causal mask
// the first min(N, (rb + 1) kSplitRows)) are cut on kSplitKeys boundaries
// into S ranges of T_rb / S tiles each (T_rb = visible keys / kSplitKeys,
// rounded up): range s is tiles [s T_rb / S, (s+1) T_rb / S).  Cutting the
// visible keys, not all N, gives every range of a causal block the same work.
// In kSplit mode a workgroup covers one (row block part, range) pair and writes,
// instead of O and L, that range's partial result: the output normalised by
// the range's own denominator, O_s (float32, [S][BH][N][d]), and the range's
// logsumexp L_s (float32, [S][BH][N]; -inf and O_s = 0 where no key of the
// range is visible to the row).  fa_merge_kernel combines them.
constexpr int kSplitRows = 256;
constexpr int kSplitKeys = 64;

// What a kernel instance does besides plain attention over all (or all
// causal) keys.
enum PathMode : int {
  kDense = 0,   // every key (or every key j <= i)
  kSplit = 1,   // one key range per workgroup, partial results (SplitArgs)
  kSparse = 2,  // only the key blocks a block mask enables (below)
  kPersist = 3, // as kDense, with each workgroup walking a list of query tiles
};

// Block-sparse attention: key j is visible to query i iff the byte
// mask[hm][i / kMaskBlock][j / kMaskBlock] is nonzero (and j <= i with the
// causal mask), hm = 0 for a mask shared by all heads, h for one mask per
// head, b*H + h for one per (batch, head).  A row with no visible key gets
// O = 0 and L = -inf.
constexpr int kMaskBlock = 64;

struct ModeArgs {
  int num_splits;             // kSplit: S (1 otherwise)
  float* opart;               // kSplit: O_s
  float* lpart;               // kSplit: L_s
  const uint8_t* mask;        // kSparse: [mask_heads][nb][nb], nb = ceil(N / 64)
  int mask_heads;             // kSparse: 1, H or B*H
  int H;                      // kSparse: heads per batch
};

// Index of the block mask of head bh (= b*H + h).
__device__ __forceinline__ int mask_head(const ModeArgs& ma, int bh) {
  return ma.mask_heads == 1 ? 0 : ma.mask_heads == ma.H ? bh % ma.H : bh;
}

// [lo, hi) of range s of row block rb.
__device__ __forceinline__ void split_range(int s, int S, int rb, int N, bool causal, int& lo,
                                            int& hi) {
  const int visible = causal ? min(N, (rb + 1) * kSplitRows) : N;
  const int T = (visible + kSplitKeys - 1) / kSplitKeys;
  lo = (s * T / S) * kSplitKeys;
  hi = min(visible, ((s + 1) * T / S) * kSplitKeys);
}

}  // namespace FA355_NS
