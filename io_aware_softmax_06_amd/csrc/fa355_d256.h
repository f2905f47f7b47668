// Host-side entry of the d = 256 kernel instances, which live in their own
// translation unit (fa355_d256.hip) built with 4-wave workgroups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Forward pass at d = 256 with 16-bit inputs (bf16 when fp16 == 0).  Without
// `opart` it writes O and L; with it (key-range split, num_splits ranges) it
// writes the partials O_s and L_s instead.  Arguments checked by the caller.
hipError_t fa355_d256_forward(const void* Q, const void* K, const void* V, void* O, float* L,
                              int64_t BH, int64_t N, float scale, int causal, int fp16,
                              int num_splits, float* opart, float* lpart, hipStream_t stream);

// Dynamic LDS bytes of one d = 256 workgroup (the K and V rings).
int fa355_d256_lds_bytes();
