// Host-side entry of the 4-wave forward instances (fa355_w4.hip): 128 query
// rows per workgroup, for launches whose 256-row tiles would leave CUs idle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Forward pass with 16-bit inputs (bf16 when fp16 == 0), d = 32, 64 or 128,
// writing O and L.  Arguments checked by the caller.
hipError_t fa355_w4_forward(const void* Q, const void* K, const void* V, void* O, float* L,
                            int64_t BH, int64_t N, int64_t d, float scale, int causal, int fp16,
                            hipStream_t stream);

// Query rows per workgroup of these instances.
int fa355_w4_rows();
