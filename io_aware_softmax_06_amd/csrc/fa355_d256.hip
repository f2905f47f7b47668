// Head dimension 256: the forward kernel built with 4-wave workgroups of 128
// query rows, one wave per SIMD (its operands and accumulators need about 300
// registers per lane), a K ring of 3 and a V ring of 2 tiles of 32 KB (the
// whole 160 KB of LDS).  A namespace of its own keeps these instances apart
// from the 8-wave ones of fa355.hip.
#define FA355_NS fa355_d256
#define FA355_BF16_WAVES 4
#define FA355_BF16_STAGES 3
#define FA355_BF16_VSTAGES 2
#define FA355_BF16_OCCUPANCY 1

// O is staged in the ring memory after the last loads (no LDS to spare).
#define FA355_STAGE_DEDICATED 0
#include "fa_fwd_bf16.hpp"
#include "fa355_d256.h"

namespace {

constexpr int kD = 256;

template <bool CAUSAL, int MODE, typename T>
hipError_t launch(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                  int64_t N, float scale, fa355_d256::ModeArgs ma, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa355_d256::fa_fwd_bf16_kernel<kD, CAUSAL, MODE, T>),
      hipFuncAttributeMaxDynamicSharedMemorySize, fa355_d256::Bf16Layout<kD>::kBytes);
  if (attr != hipSuccess) return attr;
  const int num_qtiles = (int)((N + fa355_d256::kBM - 1) / fa355_d256::kBM);
  const int total = (int)(BH * num_qtiles * ma.num_splits);
  const unsigned lds = fa355_d256::Bf16Layout<kD>::kBytes;
  hipLaunchKernelGGL((fa355_d256::fa_fwd_bf16_kernel<kD, CAUSAL, MODE, T>), dim3(total),
                     dim3(fa355_d256::kThreads), lds, s, static_cast<const uint16_t*>(Q),
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                     static_cast<uint16_t*>(O), L, (int)N, (int)BH, num_qtiles, scale,
                     scale * fa355_d256::kLog2e, ma);
  return hipGetLastError();
}

template <int MODE, typename T>
hipError_t launch_c(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                    int64_t N, float scale, int causal, fa355_d256::ModeArgs ma, hipStream_t s) {
  return causal ? launch<true, MODE, T>(Q, K, V, O, L, BH, N, scale, ma, s)
                : launch<false, MODE, T>(Q, K, V, O, L, BH, N, scale, ma, s);
}

}  // namespace

hipError_t fa355_d256_forward(const void* Q, const void* K, const void* V, void* O, float* L,
                              int64_t BH, int64_t N, float scale, int causal, int fp16,
                              int num_splits, float* opart, float* lpart, hipStream_t s) {
  const fa355_d256::ModeArgs ma = {opart ? num_splits : 1, opart, lpart, nullptr, 1, 1};
  if (opart)
    return fp16 ? launch_c<fa355_d256::kSplit, _Float16>(Q, K, V, O, L, BH, N, scale, causal, ma, s)
                : launch_c<fa355_d256::kSplit, __bf16>(Q, K, V, O, L, BH, N, scale, causal, ma, s);
  return fp16 ? launch_c<fa355_d256::kDense, _Float16>(Q, K, V, O, L, BH, N, scale, causal, ma, s)
              : launch_c<fa355_d256::kDense, __bf16>(Q, K, V, O, L, BH, N, scale, causal, ma, s);
}

int fa355_d256_lds_bytes() { return fa355_d256::Bf16Layout<kD>::kBytes; }
