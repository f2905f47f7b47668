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

#include "fa_fwd_bf16.hpp"
#include "fa_fwd_f32.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// The bf16 kernels use more than the default 64 KB of dynamic LDS; raise each
// instance's limit once per process (device-independent attribute).
template <int D, bool CAUSAL>
hipError_t prepare_bf16() {
  static const hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa355::fa_fwd_bf16_kernel<D, CAUSAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, fa355::Bf16Layout<D>::kBytes);
  return status;
}

template <int D, bool CAUSAL>
hipError_t launch_bf16(const void* Q, const void* K, const void* V, void* O, float* L,
                       int64_t BH, int64_t N, float scale, hipStream_t stream) {
  const hipError_t prep = prepare_bf16<D, CAUSAL>();
  if (prep != hipSuccess) return prep;
  const int num_qtiles = (int)((N + fa355::kBM - 1) / fa355::kBM);
  const int total = (int)(BH * num_qtiles);
  hipLaunchKernelGGL((fa355::fa_fwd_bf16_kernel<D, CAUSAL>), dim3(total), dim3(fa355::kThreads),
                     fa355::Bf16Layout<D>::kBytes, stream, static_cast<const uint16_t*>(Q),
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                     static_cast<uint16_t*>(O), L, (int)N, (int)BH, num_qtiles, scale,
                     scale * fa355::kLog2e);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                int64_t N, float scale, hipStream_t stream) {
  constexpr int kRows = 64 / (D / 64);
  const int num_qtiles = (int)((N + kRows - 1) / kRows);
  const int total = (int)(BH * num_qtiles);
  hipLaunchKernelGGL((fa355::fa_fwd_f32_kernel<D, CAUSAL>), dim3(total), dim3(64), 0, stream,
                     static_cast<const float*>(Q), static_cast<const float*>(K),
                     static_cast<const float*>(V), static_cast<float*>(O), L, (int)N, num_qtiles,
                     scale, scale * fa355::kLog2e);
  return hipGetLastError();
}

}  // namespace

extern "C" int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int64_t B,
                      int64_t H, int64_t N, int64_t d, float scale, int causal, void* stream,
                      int dtype) {
  if (!Q || !K || !V || !O || !L) return FA_ERR_NULL;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;

  // Index ranges: rows are int inside the kernels, workgroup counts must fit
  // a 32-bit grid, byte sizes must fit 64 bits.
  if (N > INT_MAX - 256 || B > INT_MAX || H > INT_MAX) return FA_ERR_SHAPE;
  const int64_t BH = B * H;
  if (BH > INT_MAX) return FA_ERR_SHAPE;
  const int64_t min_rows_per_block = 32;
  if (BH * ((N + min_rows_per_block - 1) / min_rows_per_block) > INT_MAX) return FA_ERR_SHAPE;
  const uint64_t esize = dtype == FA_BF16 ? 2 : 4;
  const uint64_t rows = (uint64_t)BH * (uint64_t)N;
  if (rows > (UINT64_MAX / 4) / ((uint64_t)d * esize)) return FA_ERR_SHAPE;
  const uint64_t tensor_bytes = rows * (uint64_t)d * esize;
  const uint64_t lse_bytes = rows * 4;

  const uintptr_t misalign = reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) |
                             reinterpret_cast<uintptr_t>(V) | reinterpret_cast<uintptr_t>(O);
  if ((misalign & 15u) != 0 || (reinterpret_cast<uintptr_t>(L) & 3u) != 0) return FA_ERR_ALIGN;

  for (const void* in : {Q, K, V}) {
    if (ranges_overlap(O, tensor_bytes, in, tensor_bytes)) return FA_ERR_ALIAS;
    if (ranges_overlap(L, lse_bytes, in, tensor_bytes)) return FA_ERR_ALIAS;
  }
  if (ranges_overlap(L, lse_bytes, O, tensor_bytes)) return FA_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear an error left by an earlier, unrelated call
  hipError_t err;
  if (dtype == FA_BF16) {
    if (d == 64)
      err = causal ? launch_bf16<64, true>(Q, K, V, O, L, BH, N, scale, s)
                   : launch_bf16<64, false>(Q, K, V, O, L, BH, N, scale, s);
    else
      err = causal ? launch_bf16<128, true>(Q, K, V, O, L, BH, N, scale, s)
                   : launch_bf16<128, false>(Q, K, V, O, L, BH, N, scale, s);
  } else {
    if (d == 64)
      err = causal ? launch_f32<64, true>(Q, K, V, O, L, BH, N, scale, s)
                   : launch_f32<64, false>(Q, K, V, O, L, BH, N, scale, s);
    else
      err = causal ? launch_f32<128, true>(Q, K, V, O, L, BH, N, scale, s)
                   : launch_f32<128, false>(Q, K, V, O, L, BH, N, scale, s);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is < 1 or too large to index";
    case FA_ERR_UNSUPPORTED_D: return "head dimension d must be 64 or 128";
    case FA_ERR_DTYPE: return "dtype must be FA_BF16 (0) or FA_F32 (1)";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIGN: return "Q, K, V, O must be 16-byte aligned and L 4-byte aligned";
    case FA_ERR_ALIAS: return "O or L overlaps an input, or O overlaps L";
    case FA_ERR_HIP: return "the HIP runtime reported an error at kernel launch";
    case FA_ERR_ARG: return "causal must be 0 or 1";
    default: return "unknown status code";
  }
}

extern "C" int fa_version(void) { return kVersion; }
