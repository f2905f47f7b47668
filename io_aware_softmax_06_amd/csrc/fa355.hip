// libfa355: host side of the C ABI declared in include/fa355.h.
//
// Checks every argument on the host before any HIP runtime call, picks the
// kernel instance for (dtype, d, causal) and enqueues it on the caller's
// stream.  No device memory is allocated here.
#include "fa355.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_fwd_bf16.hpp"
#include "fa_fwd_f32.hpp"
#include "fa_merge.hpp"
#include "fa_bwd_bf16.hpp"
#include "fa_bwd_f32.hpp"
#include "fa355_d256.h"
#include "fa355_w4.h"

namespace {

constexpr int kVersion = 600;  // 0.6.0: fa_fwd_splitkv_noalloc
constexpr int kMaxSplits = 128;
constexpr int kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Sizes derived from a validated call.
struct Sizes {
  int64_t BH;
  uint64_t rows;          // B*H*N
  uint64_t tensor_bytes;  // one of Q, K, V, O
  uint64_t lse_bytes;     // L
};

// Every check of fa_fwd, before any HIP call.  Returns FA_OK or the status.
int check_args(const void* Q, const void* K, const void* V, void* O, float* L, int64_t B,
               int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, Sizes* sz) {
  if (!Q || !K || !V || !O || !L) return FA_ERR_NULL;
  if (dtype != FA_BF16 && dtype != FA_F32 && dtype != FA_F16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED_D;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;

  // Index ranges: rows are int inside the kernels, workgroup counts must fit
  // a 32-bit grid, byte sizes must fit 64 bits.
  if (N > INT_MAX - 256 || B > INT_MAX || H > INT_MAX) return FA_ERR_SHAPE;
  const int64_t BH = B * H;
  if (BH > INT_MAX) return FA_ERR_SHAPE;
  const int64_t min_rows_per_block = 32;
  if (BH * ((N + min_rows_per_block - 1) / min_rows_per_block) > INT_MAX) return FA_ERR_SHAPE;
  const uint64_t esize = dtype == FA_F32 ? 4 : 2;
  const uint64_t rows = (uint64_t)BH * (uint64_t)N;
  if (rows > (UINT64_MAX / 4) / ((uint64_t)d * esize)) return FA_ERR_SHAPE;
  const uint64_t tensor_bytes = rows * (uint64_t)d * esize;
  // The 16-bit kernels read K and V through buffer resources whose size field
  // holds one head (N * d * 2 bytes) as a 32-bit signed count.
  if (dtype != FA_F32 && (uint64_t)N * (uint64_t)d * 2 > (uint64_t)INT_MAX) return FA_ERR_SHAPE;
  const uint64_t lse_bytes = rows * 4;

  const uintptr_t misalign = reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) |
                             reinterpret_cast<uintptr_t>(V) | reinterpret_cast<uintptr_t>(O);
  if ((misalign & 15u) != 0 || (reinterpret_cast<uintptr_t>(L) & 3u) != 0) return FA_ERR_ALIGN;

  for (const void* in : {Q, K, V}) {
    if (ranges_overlap(O, tensor_bytes, in, tensor_bytes)) return FA_ERR_ALIAS;
    if (ranges_overlap(L, lse_bytes, in, tensor_bytes)) return FA_ERR_ALIAS;
  }
  if (ranges_overlap(L, lse_bytes, O, tensor_bytes)) return FA_ERR_ALIAS;
  *sz = {BH, rows, tensor_bytes, lse_bytes};
  return FA_OK;
}

// Workspace of the split forward: O_s (float32 [S][rows][d]) then L_s
// (float32 [S][rows]).  0 if the size does not fit 64 bits.
uint64_t split_workspace_bytes(uint64_t rows, int64_t d, int splits) {
  const uint64_t per_split = rows * ((uint64_t)d + 1) * 4;
  if (per_split > UINT64_MAX / (uint64_t)splits) return 0;
  return per_split * (uint64_t)splits;
}

// The bf16 kernels use more than the default 64 KB of dynamic LDS; raise each
// instance's limit once per process (device-independent attribute).
// Dynamic LDS of a bf16 launch: the K and V rings, plus on the block-sparse
// path the tile list (one word per key block) and one count per wave.
// Dense and persistent launches also hold the output staging area past the
// rings.
template <int D, int MODE>
int64_t bf16_lds_bytes(int64_t N) {
  using Lay = fa355::Bf16Layout<D>;
  if (MODE == fa355::kSparse)
    return Lay::kBytes + 4 * ((N + fa355::kMaskBlock - 1) / fa355::kMaskBlock + fa355::kWaves);
  return MODE == fa355::kSplit ? Lay::kBytes : Lay::kBytesStaged;
}

// The bf16 kernels use more than the default 64 KB of dynamic LDS; raise each
// instance's limit once per process (device-independent attribute) to what
// its largest launch may use.
template <int D, bool CAUSAL, int MODE, typename T>
hipError_t prepare_bf16() {
  static const hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa355::fa_fwd_bf16_kernel<D, CAUSAL, MODE, T>),
      hipFuncAttributeMaxDynamicSharedMemorySize,
      MODE == fa355::kSparse ? kMaxLds : (int)bf16_lds_bytes<D, MODE>(0));
  return status;
}

#ifndef FA355_PERSIST
#define FA355_PERSIST 1
#endif
#ifndef FA355_W4
#define FA355_W4 1
#endif

// Compute units of the current device (0 if the query fails), cached per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cached[dev] = n > 0 ? n : 0;
  }
  return cached[dev];
}

// Workgroups of a persistent dense launch: one per CU (a workgroup fills a
// CU), at most one per query tile, and a multiple of the 8 XCDs when the heads
// split evenly over them, so that every XCD serves its own heads.
int persist_grid(int64_t BH, int items, int cus) {
  int grid = items < cus ? items : cus;
  if (BH % 8 == 0 && grid >= 8) grid -= grid % 8;
  return grid;
}

template <int D, bool CAUSAL, int MODE, typename T>
hipError_t launch_bf16(const void* Q, const void* K, const void* V, void* O, float* L,
                       int64_t BH, int64_t N, float scale, fa355::ModeArgs sa,
                       hipStream_t stream) {
  const int num_qtiles = (int)((N + fa355::kBM - 1) / fa355::kBM);
  // Causal only: measured on non-causal workloads the persistent launch was
  // 1-2% slower than hardware dispatch of one workgroup per query tile.
  if constexpr (MODE == fa355::kDense && CAUSAL && FA355_PERSIST) {
    const int items = (int)(BH * num_qtiles);
    const int cus = device_cus();
    // The ring carried from one query tile to the next holds that tile's first
    // kStages key tiles: every query tile must stream at least that many.
    if (cus > 0 && items > cus && N > (int64_t)(fa355::kStages - 1) * fa355::kBN)
      return launch_bf16<D, CAUSAL, fa355::kPersist, T>(Q, K, V, O, L, BH, N, scale, sa, stream);
  }
  const hipError_t prep = prepare_bf16<D, CAUSAL, MODE, T>();
  if (prep != hipSuccess) return prep;
  int total = (int)(BH * num_qtiles * sa.num_splits);
  if (MODE == fa355::kPersist) total = persist_grid(BH, total, device_cus());
  const unsigned lds = (unsigned)bf16_lds_bytes<D, MODE>(N);
  hipLaunchKernelGGL((fa355::fa_fwd_bf16_kernel<D, CAUSAL, MODE, T>), dim3(total),
                     dim3(fa355::kThreads), lds, stream,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), static_cast<uint16_t*>(O), L, (int)N,
                     (int)BH, num_qtiles, scale, scale * fa355::kLog2e, sa);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int MODE>
hipError_t launch_f32(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                      int64_t N, float scale, fa355::ModeArgs sa, hipStream_t stream) {
  constexpr int kRows = fa355::kF32Rows;  // query rows per workgroup
  const int num_qtiles = (int)((N + kRows - 1) / kRows);
  const int total = (int)(BH * num_qtiles * sa.num_splits);
  hipLaunchKernelGGL((fa355::fa_fwd_f32_kernel<D, CAUSAL, MODE>), dim3(total), dim3(64), 0,
                     stream, static_cast<const float*>(Q), static_cast<const float*>(K),
                     static_cast<const float*>(V), static_cast<float*>(O), L, (int)N, (int)BH,
                     num_qtiles, scale, scale * fa355::kLog2e, sa);
  return hipGetLastError();
}

template <int MODE, typename T>
hipError_t launch_mfma(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                       int64_t N, int64_t d, float scale, int causal, fa355::ModeArgs sa,
                       hipStream_t s) {
  if (d == 32)
    return causal ? launch_bf16<32, true, MODE, T>(Q, K, V, O, L, BH, N, scale, sa, s)
                  : launch_bf16<32, false, MODE, T>(Q, K, V, O, L, BH, N, scale, sa, s);
  if (d == 64)
    return causal ? launch_bf16<64, true, MODE, T>(Q, K, V, O, L, BH, N, scale, sa, s)
                  : launch_bf16<64, false, MODE, T>(Q, K, V, O, L, BH, N, scale, sa, s);
  return causal ? launch_bf16<128, true, MODE, T>(Q, K, V, O, L, BH, N, scale, sa, s)
                : launch_bf16<128, false, MODE, T>(Q, K, V, O, L, BH, N, scale, sa, s);
}

template <int MODE>
hipError_t launch_forward(const void* Q, const void* K, const void* V, void* O, float* L,
                          int64_t BH, int64_t N, int64_t d, float scale, int causal, int dtype,
                          fa355::ModeArgs sa, hipStream_t s) {
  if (d == 256 && dtype != FA_F32) {
    return fa355_d256_forward(Q, K, V, O, L, BH, N, scale, causal, dtype == FA_F16 ? 1 : 0,
                              sa.num_splits, MODE == fa355::kSplit ? sa.opart : nullptr,
                              sa.lpart, s);
  }
  if (d == 256)
    return causal ? launch_f32<256, true, MODE>(Q, K, V, O, L, BH, N, scale, sa, s)
                  : launch_f32<256, false, MODE>(Q, K, V, O, L, BH, N, scale, sa, s);
  // Dense 16-bit launches whose 256-row tiles would leave CUs idle take the
  // 128-row build (fa355_w4.hip): fewer tiles than CUs, or, under the causal
  // mask, where the longest tile sets the time, no more tiles than CUs.
  if constexpr (MODE == fa355::kDense && FA355_W4) {
    if (dtype != FA_F32) {
      const int cus = device_cus();
      const int64_t tiles = BH * ((N + fa355::kBM - 1) / fa355::kBM);
      if (cus > 0 && (tiles < cus || (causal && tiles <= cus)))
        return fa355_w4_forward(Q, K, V, O, L, BH, N, d, scale, causal, dtype == FA_F16 ? 1 : 0,
                                s);
    }
  }
  if (dtype == FA_BF16) return launch_mfma<MODE, __bf16>(Q, K, V, O, L, BH, N, d, scale, causal, sa, s);
  if (dtype == FA_F16) return launch_mfma<MODE, _Float16>(Q, K, V, O, L, BH, N, d, scale, causal, sa, s);
  if (d == 32)
    return causal ? launch_f32<32, true, MODE>(Q, K, V, O, L, BH, N, scale, sa, s)
                  : launch_f32<32, false, MODE>(Q, K, V, O, L, BH, N, scale, sa, s);
  if (d == 64)
    return causal ? launch_f32<64, true, MODE>(Q, K, V, O, L, BH, N, scale, sa, s)
                  : launch_f32<64, false, MODE>(Q, K, V, O, L, BH, N, scale, sa, s);
  return causal ? launch_f32<128, true, MODE>(Q, K, V, O, L, BH, N, scale, sa, s)
                : launch_f32<128, false, MODE>(Q, K, V, O, L, BH, N, scale, sa, s);
}

template <int D, typename OutT>
hipError_t launch_merge(const float* opart, const float* lpart, void* O, float* L, int S,
                        uint64_t rows, hipStream_t s) {
  constexpr int kRowsPerBlock = fa355::kMergeThreads / (D / 4);
  constexpr uint64_t kMaxBlocks = 1u << 20;  // the kernel strides over the rest
  uint64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  hipLaunchKernelGGL((fa355::fa_merge_kernel<D, OutT>), dim3((unsigned)blocks),
                     dim3(fa355::kMergeThreads), 0, s, opart, lpart, static_cast<OutT*>(O), L, S,
                     (int64_t)rows);
  return hipGetLastError();
}

template <typename OutT>
hipError_t launch_merge_d(const float* opart, const float* lpart, void* O, float* L, int S,
                          uint64_t rows, int64_t d, hipStream_t s) {
  if (d == 32) return launch_merge<32, OutT>(opart, lpart, O, L, S, rows, s);
  if (d == 256) return launch_merge<256, OutT>(opart, lpart, O, L, S, rows, s);
  if (d == 64) return launch_merge<64, OutT>(opart, lpart, O, L, S, rows, s);
  return launch_merge<128, OutT>(opart, lpart, O, L, S, rows, s);
}

}  // namespace

extern "C" int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int64_t B,
                      int64_t H, int64_t N, int64_t d, float scale, int causal, void* stream,
                      int dtype) {
  Sizes sz;
  const int rc = check_args(Q, K, V, O, L, B, H, N, d, scale, causal, dtype, &sz);
  if (rc != FA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear an error left by an earlier, unrelated call
  const fa355::ModeArgs whole = {1, nullptr, nullptr, nullptr, 1, (int)H};
  const hipError_t err =
      launch_forward<fa355::kDense>(Q, K, V, O, L, sz.BH, N, d, scale, causal, dtype, whole, s);
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int64_t fa_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t d,
                                            int num_splits) {
  if (B < 1 || H < 1 || N < 1 || B > INT_MAX || H > INT_MAX || N > INT_MAX - 256)
    return FA_ERR_SHAPE;
  if (B * H > INT_MAX) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED_D;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_SPLITS;
  const uint64_t bytes = split_workspace_bytes((uint64_t)(B * H) * (uint64_t)N, d, num_splits);
  if (bytes == 0 || bytes > (uint64_t)INT64_MAX) return FA_ERR_SHAPE;
  return (int64_t)bytes;
}

namespace {

// The split forward on a given workspace (fa_fwd_splitkv's checks and
// launches); `workspace` is device memory of at least `workspace_bytes`.
int splitkv_impl(const void* Q, const void* K, const void* V, void* O, float* L, int64_t B,
                 int64_t H, int64_t N, int64_t d, float scale, int causal, void* stream,
                 int dtype, int num_splits, void* workspace, int64_t workspace_bytes) {
  Sizes sz;
  const int rc = check_args(Q, K, V, O, L, B, H, N, d, scale, causal, dtype, &sz);
  if (rc != FA_OK) return rc;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_SPLITS;
  // Grid of the split pass: one workgroup per (query tile, split) of each head.
  const int64_t min_rows_per_block = 32;
  if (sz.BH * ((N + min_rows_per_block - 1) / min_rows_per_block) * num_splits > INT_MAX)
    return FA_ERR_SHAPE;
  const uint64_t need = split_workspace_bytes(sz.rows, d, num_splits);
  if (need == 0) return FA_ERR_SHAPE;
  if (!workspace || workspace_bytes < 0 || (uint64_t)workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return FA_ERR_WORKSPACE;
  for (const void* p : {Q, K, V, static_cast<const void*>(O)})
    if (ranges_overlap(workspace, need, p, sz.tensor_bytes)) return FA_ERR_ALIAS;
  if (ranges_overlap(workspace, need, L, sz.lse_bytes)) return FA_ERR_ALIAS;

  float* opart = static_cast<float*>(workspace);
  float* lpart = opart + sz.rows * (uint64_t)d * (uint64_t)num_splits;
  const fa355::ModeArgs sa = {num_splits, opart, lpart, nullptr, 1, (int)H};

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t err =
      launch_forward<fa355::kSplit>(Q, K, V, O, L, sz.BH, N, d, scale, causal, dtype, sa, s);
  if (err == hipSuccess) {
    if (dtype == FA_BF16)
      err = launch_merge_d<__bf16>(opart, lpart, O, L, num_splits, sz.rows, d, s);
    else if (dtype == FA_F16)
      err = launch_merge_d<_Float16>(opart, lpart, O, L, num_splits, sz.rows, d, s);
    else
      err = launch_merge_d<float>(opart, lpart, O, L, num_splits, sz.rows, d, s);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* L,
                              int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                              void* stream, int dtype, int num_splits, void* workspace,
                              int64_t workspace_bytes) {
  return splitkv_impl(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype, num_splits,
                      workspace, workspace_bytes);
}

// The library's own split workspace for callers that cannot allocate: one
// copy per device, held while the process lives.  In host code this name is
// a host-side stand-in, not a device address; the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device (resolved on the first
// call on that device, with it current), or nullptr if that failed.
void* scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) addr[dev] = p;
  });
  return addr[dev];
}

}  // namespace

extern "C" int fa_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O,
                                      float* L, int64_t B, int64_t H, int64_t N, int64_t d,
                                      float scale, int causal, void* stream, int dtype,
                                      int num_splits) {
  // Sizes first, so that every rejection happens before any HIP call.
  Sizes sz;
  const int rc = check_args(Q, K, V, O, L, B, H, N, d, scale, causal, dtype, &sz);
  if (rc != FA_OK) return rc;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_SPLITS;
  const uint64_t need = split_workspace_bytes(sz.rows, d, num_splits);
  if (need == 0) return FA_ERR_SHAPE;
  if (need > (uint64_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return FA_ERR_HIP;
  return splitkv_impl(Q, K, V, O, L, B, H, N, d, scale, causal, stream, dtype, num_splits, ws,
                      (int64_t)FA_NOALLOC_SCRATCH_BYTES);
}

extern "C" int fa_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* L,
                                  int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                  int causal, void* stream, int dtype, const uint8_t* block_mask,
                                  int64_t mask_heads) {
  Sizes sz;
  const int rc = check_args(Q, K, V, O, L, B, H, N, d, scale, causal, dtype, &sz);
  if (rc != FA_OK) return rc;
  if (d == 256) return FA_ERR_UNSUPPORTED_D;  // the rings fill the LDS: no room for the list
  if (!block_mask) return FA_ERR_NULL;
  if (mask_heads != 1 && mask_heads != H && mask_heads != sz.BH) return FA_ERR_ARG;
  const int64_t nb = (N + fa355::kMaskBlock - 1) / fa355::kMaskBlock;
  // The tile list lives in LDS next to the K and V rings.
  const int64_t lds = d == 32   ? bf16_lds_bytes<32, fa355::kSparse>(N)
                      : d == 64 ? bf16_lds_bytes<64, fa355::kSparse>(N)
                                : bf16_lds_bytes<128, fa355::kSparse>(N);
  if (dtype != FA_F32 && lds > kMaxLds) return FA_ERR_SHAPE;
  const uint64_t mask_bytes = (uint64_t)mask_heads * (uint64_t)nb * (uint64_t)nb;
  if (ranges_overlap(block_mask, mask_bytes, O, sz.tensor_bytes) ||
      ranges_overlap(block_mask, mask_bytes, L, sz.lse_bytes))
    return FA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const fa355::ModeArgs ma = {1, nullptr, nullptr, block_mask, (int)mask_heads, (int)H};
  const hipError_t err =
      launch_forward<fa355::kSparse>(Q, K, V, O, L, sz.BH, N, d, scale, causal, dtype, ma, s);
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Backward pass.

template <int D, bool CAUSAL, typename T>
hipError_t launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* Dv, void* dQ, void* dK, void* dV,
                           int64_t BH, int64_t N, float scale, hipStream_t s) {
  static const hipError_t attr_kv = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa355::fa_bwd_dkdv_bf16_kernel<D, CAUSAL, T>),
      hipFuncAttributeMaxDynamicSharedMemorySize, fa355::BwdKvLayout<D>::kBytes);
  static const hipError_t attr_q = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa355::fa_bwd_dq_bf16_kernel<D, CAUSAL, T>),
      hipFuncAttributeMaxDynamicSharedMemorySize, fa355::BwdQLayout<D>::kBytes);
  if (attr_kv != hipSuccess) return attr_kv;
  if (attr_q != hipSuccess) return attr_q;
  const float c = scale * fa355::kLog2e;
  const auto* q = static_cast<const uint16_t*>(Q);
  const auto* k = static_cast<const uint16_t*>(K);
  const auto* v = static_cast<const uint16_t*>(V);
  const auto* g = static_cast<const uint16_t*>(dO);
  const int nk = (int)((N + fa355::kBwdKvKeys - 1) / fa355::kBwdKvKeys);
  const unsigned lds_kv = fa355::BwdKvLayout<D>::kBytes, lds_q = fa355::BwdQLayout<D>::kBytes;
  hipLaunchKernelGGL((fa355::fa_bwd_dkdv_bf16_kernel<D, CAUSAL, T>), dim3((unsigned)(BH * nk)),
                     dim3(64 * fa355::kBwdKvWaves), lds_kv, s, q, k, v, g, L, Dv,
                     static_cast<uint16_t*>(dK), static_cast<uint16_t*>(dV), (int)N, (int)BH, scale,
                     c);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nq = (int)((N + fa355::kBM - 1) / fa355::kBM);
  hipLaunchKernelGGL((fa355::fa_bwd_dq_bf16_kernel<D, CAUSAL, T>), dim3((unsigned)(BH * nq)),
                     dim3(fa355::kThreads), lds_q, s, q, k, v, g, L, Dv,
                     static_cast<uint16_t*>(dQ), (int)N, (int)BH, nq, scale, c);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_f32(const void* Q, const void* K, const void* V, const void* dO,
                          const float* L, const float* Dv, void* dQ, void* dK, void* dV,
                          int64_t BH, int64_t N, float scale, hipStream_t s) {
  constexpr int kRows = D >= 64 ? 64 / (D / 64) : 64;
  const float c = scale * fa355::kLog2e;
  const auto* q = static_cast<const float*>(Q);
  const auto* k = static_cast<const float*>(K);
  const auto* v = static_cast<const float*>(V);
  const auto* g = static_cast<const float*>(dO);
  const int nt = (int)((N + kRows - 1) / kRows);
  hipLaunchKernelGGL((fa355::fa_bwd_dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)(BH * nt)),
                     dim3(64), 0, s, q, k, v, g, L, Dv, static_cast<float*>(dK),
                     static_cast<float*>(dV), (int)N, nt, scale, c);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((fa355::fa_bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)(BH * nt)),
                     dim3(64), 0, s, q, k, v, g, L, Dv, static_cast<float*>(dQ), (int)N, nt, scale,
                     c);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_bwd_dot(const void* O, const void* dO, float* Dv, uint64_t rows, hipStream_t s) {
  constexpr int kRowsPer = fa355::kDotThreads / (D / 8);
  uint64_t blocks = (rows + kRowsPer - 1) / kRowsPer;
  if (blocks > (1u << 20)) blocks = 1u << 20;
  hipLaunchKernelGGL((fa355::fa_bwd_dot_kernel<D, T>), dim3((unsigned)blocks),
                     dim3(fa355::kDotThreads), 0, s, static_cast<const T*>(O),
                     static_cast<const T*>(dO), Dv, (int64_t)rows);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_mfma(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* L, float* Dv, void* dQ, void* dK, void* dV,
                           const Sizes& sz, int64_t N, int64_t d, float scale, int causal,
                           hipStream_t s) {
  hipError_t err = d == 32   ? launch_bwd_dot<32, T>(O, dO, Dv, sz.rows, s)
                   : d == 64 ? launch_bwd_dot<64, T>(O, dO, Dv, sz.rows, s)
                             : launch_bwd_dot<128, T>(O, dO, Dv, sz.rows, s);
  if (err != hipSuccess) return err;
  if (d == 32)
    return causal ? launch_bwd_bf16<32, true, T>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s)
                  : launch_bwd_bf16<32, false, T>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s);
  if (d == 64)
    return causal ? launch_bwd_bf16<64, true, T>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s)
                  : launch_bwd_bf16<64, false, T>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s);
  return causal ? launch_bwd_bf16<128, true, T>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s)
                : launch_bwd_bf16<128, false, T>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s);
}

extern "C" int64_t fa_bwd_workspace(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 1 || H < 1 || N < 1 || B > INT_MAX || H > INT_MAX || N > INT_MAX - 256)
    return FA_ERR_SHAPE;
  if (B * H > INT_MAX) return FA_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;  // backward: d <= 128
  // B*H and N are each below 2^31, so the row count fits 62 bits; four bytes
  // per row must still fit a signed 64-bit result.
  const uint64_t rows = (uint64_t)(B * H) * (uint64_t)N;
  if (rows > (uint64_t)INT64_MAX / 4) return FA_ERR_SHAPE;
  return (int64_t)(rows * 4);
}

extern "C" int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* L, void* dQ, void* dK, void* dV, int64_t B, int64_t H,
                      int64_t N, int64_t d, float scale, int causal, void* stream, int dtype,
                      void* workspace, int64_t workspace_bytes) {
  if (!dO || !dQ || !dK || !dV) return FA_ERR_NULL;
  // fa_fwd's checks with O and L as the "outputs": shapes, dtype, scale,
  // causal, alignment of Q, K, V, O and L, and no overlap of O or L with
  // Q, K, V.
  Sizes sz;
  const int rc = check_args(Q, K, V, const_cast<void*>(O), const_cast<float*>(L), B, H, N, d,
                            scale, causal, dtype, &sz);
  if (rc != FA_OK) return rc;
  if (d == 256) return FA_ERR_UNSUPPORTED_D;  // backward: d <= 128
  const uintptr_t misalign = reinterpret_cast<uintptr_t>(dO) | reinterpret_cast<uintptr_t>(dQ) |
                             reinterpret_cast<uintptr_t>(dK) | reinterpret_cast<uintptr_t>(dV);
  if ((misalign & 15u) != 0) return FA_ERR_ALIGN;
  const uint64_t need = sz.rows * 4;
  if (!workspace || workspace_bytes < 0 || (uint64_t)workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return FA_ERR_WORKSPACE;
  // Every written buffer (dQ, dK, dV, workspace) overlaps no other buffer.
  const void* outs[4] = {dQ, dK, dV, workspace};
  const uint64_t out_bytes[4] = {sz.tensor_bytes, sz.tensor_bytes, sz.tensor_bytes, need};
  const void* ins[6] = {Q, K, V, O, dO, L};
  const uint64_t in_bytes[6] = {sz.tensor_bytes, sz.tensor_bytes, sz.tensor_bytes,
                                sz.tensor_bytes, sz.tensor_bytes, sz.lse_bytes};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (ranges_overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (ranges_overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA_ERR_ALIAS;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  float* Dv = static_cast<float*>(workspace);
  hipError_t err;
  if (dtype == FA_BF16)
    err = launch_bwd_mfma<__bf16>(Q, K, V, O, dO, L, Dv, dQ, dK, dV, sz, N, d, scale, causal, s);
  else if (dtype == FA_F16)
    err = launch_bwd_mfma<_Float16>(Q, K, V, O, dO, L, Dv, dQ, dK, dV, sz, N, d, scale, causal, s);
  else {
    err = d == 32   ? launch_bwd_dot<32, float>(O, dO, Dv, sz.rows, s)
          : d == 64 ? launch_bwd_dot<64, float>(O, dO, Dv, sz.rows, s)
                    : launch_bwd_dot<128, float>(O, dO, Dv, sz.rows, s);
    if (err == hipSuccess) {
      if (d == 32)
        err = causal ? launch_bwd_f32<32, true>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s)
                     : launch_bwd_f32<32, false>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s);
      else if (d == 64)
        err = causal ? launch_bwd_f32<64, true>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s)
                     : launch_bwd_f32<64, false>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s);
      else
        err = causal ? launch_bwd_f32<128, true>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s)
                     : launch_bwd_f32<128, false>(Q, K, V, dO, L, Dv, dQ, dK, dV, sz.BH, N, scale, s);
    }
  }
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is < 1 or too large to index";
    case FA_ERR_UNSUPPORTED_D: return "head dimension d must be 32, 64, 128 or 256 (the "
                                      "backward and block-sparse paths: 32, 64 or 128)";
    case FA_ERR_DTYPE: return "dtype must be FA_BF16 (0), FA_F32 (1) or FA_F16 (2)";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIGN: return "Q, K, V, O must be 16-byte aligned and L 4-byte aligned";
    case FA_ERR_ALIAS: return "O, L or the workspace overlaps another buffer of the call";
    case FA_ERR_HIP: return "the HIP runtime reported an error at kernel launch";
    case FA_ERR_ARG: return "causal must be 0 or 1";
    case FA_ERR_SPLITS: return "num_splits must be between 1 and 128";
    case FA_ERR_WORKSPACE: return "workspace is NULL, smaller than fa_fwd_splitkv_workspace() "
                                  "bytes or not 256-byte aligned";
    case FA_ERR_SCRATCH: return "the split workspace this call needs exceeds the library's "
                                "fixed scratch buffer (FA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status code";
  }
}

extern "C" int fa_version(void) { return kVersion; }
