// The forward kernel built with 4-wave workgroups of 128 query rows, two
// waves per SIMD as in the 8-wave build, and a K ring of 3 and a V ring of 2
// tiles (80 KB of LDS at d = 128), so that two workgroups share a CU.  Twice
// as many workgroups cover the same rows: launches with fewer 256-row tiles
// than CUs fill the chip, and causal launches, whose longest tile sets the
// time, get tiles half as long.  On launches that fill the chip anyway the
// 8-wave build is faster (each workgroup fills its own K and V tiles, so LDS
// fills and L2 reads double).  A namespace of its own keeps these instances
// apart from the 8-wave ones of fa355.hip.
#define FA355_NS fa355_w4
#define FA355_BF16_WAVES 4
#define FA355_BF16_STAGES 3
#define FA355_BF16_VSTAGES 2
#define FA355_BF16_OCCUPANCY 2
// O is staged in the ring memory after the last loads, keeping two
// workgroups per CU.
#define FA355_STAGE_DEDICATED 0

#include "fa_fwd_bf16.hpp"
#include "fa355_w4.h"

namespace {

template <int D, bool CAUSAL, typename T>
hipError_t launch(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                  int64_t N, float scale, hipStream_t s) {
  using Lay = fa355_w4::Bf16Layout<D>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa355_w4::fa_fwd_bf16_kernel<D, CAUSAL, fa355_w4::kDense, T>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Lay::kBytes);
  if (attr != hipSuccess) return attr;
  const int num_qtiles = (int)((N + fa355_w4::kBM - 1) / fa355_w4::kBM);
  const fa355_w4::ModeArgs ma = {1, nullptr, nullptr, nullptr, 1, 1};
  hipLaunchKernelGGL((fa355_w4::fa_fwd_bf16_kernel<D, CAUSAL, fa355_w4::kDense, T>),
                     dim3((unsigned)(BH * num_qtiles)), dim3(fa355_w4::kThreads), Lay::kBytes, s,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), static_cast<uint16_t*>(O), L, (int)N,
                     (int)BH, num_qtiles, scale, scale * fa355_w4::kLog2e, ma);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_c(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                    int64_t N, float scale, int causal, hipStream_t s) {
  return causal ? launch<D, true, T>(Q, K, V, O, L, BH, N, scale, s)
                : launch<D, false, T>(Q, K, V, O, L, BH, N, scale, s);
}

template <typename T>
hipError_t launch_d(const void* Q, const void* K, const void* V, void* O, float* L, int64_t BH,
                    int64_t N, int64_t d, float scale, int causal, hipStream_t s) {
  if (d == 32) return launch_c<32, T>(Q, K, V, O, L, BH, N, scale, causal, s);
  if (d == 64) return launch_c<64, T>(Q, K, V, O, L, BH, N, scale, causal, s);
  return launch_c<128, T>(Q, K, V, O, L, BH, N, scale, causal, s);
}

}  // namespace

hipError_t fa355_w4_forward(const void* Q, const void* K, const void* V, void* O, float* L,
                            int64_t BH, int64_t N, int64_t d, float scale, int causal, int fp16,
                            hipStream_t s) {
  return fp16 ? launch_d<_Float16>(Q, K, V, O, L, BH, N, d, scale, causal, s)
              : launch_d<__bf16>(Q, K, V, O, L, BH, N, d, scale, causal, s);
}

int fa355_w4_rows() { return fa355_w4::kBM; }
