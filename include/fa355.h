/*
 * libfa355 -- exact attention forward pass on AMD Instinct MI355X (gfx950).
 *
 * The operation is the standard scaled dot-product attention stated in
 * "理解 Flash Attention：在 Triton 中从头编写算法" (section "什么是注意力？"),
 * computed without ever writing the N x N score matrix to device memory:
 * each workgroup owns one block of query rows and streams every block of
 * keys and values past it, keeping per row a running maximum m, a running
 * softmax denominator l and an un-normalised output (the wmrh.cn article on
 * FlashAttention, section 2.2 on embedding online softmax into attention;
 * the concatenation rule in section "瓦片注意力计算" of the Triton article).
 *
 * All entry points are plain C; no C++ or framework types cross this line.
 */
#ifndef FA355_H
#define FA355_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum {
  FA_BF16 = 0, /* bfloat16 inputs and output, float32 accumulation */
  FA_F32 = 1   /* float32 inputs and output, float32 arithmetic */
} fa_dtype;

/* Status codes.  Every negative code except FA_ERR_HIP is returned by the
 * host-side argument checks, before any HIP runtime call is made. */
typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,           /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,          /* B, H or N < 1, or a size too large to index */
  FA_ERR_UNSUPPORTED_D = -3,  /* head dimension d is not 64 or 128 */
  FA_ERR_DTYPE = -4,          /* dtype is not an fa_dtype value */
  FA_ERR_SCALE = -5,          /* scale is not finite or not > 0 */
  FA_ERR_ALIGN = -6,          /* Q, K, V or O not 16-byte aligned, or L not 4-byte aligned */
  FA_ERR_ALIAS = -7,          /* O or L overlaps an input, or O overlaps L */
  FA_ERR_HIP = -8,            /* the HIP runtime reported an error at launch */
  FA_ERR_ARG = -9             /* causal is not 0 or 1 */
} fa_status;

/*
 * fa_fwd -- O = softmax(scale * Q K^T [+ causal mask]) V and its logsumexp L.
 *
 *   Q, K, V  device pointers to [B, H, N, d] tensors, contiguous row-major
 *            (d fastest), element type `dtype`.  Read only.
 *   O        device pointer, [B, H, N, d], element type `dtype`.  Written.
 *   L        device pointer, [B, H, N] float32.  Written with the natural-log
 *            logsumexp of each row's scaled, masked scores:
 *            L[b,h,i] = ln sum_j exp(scale * q_i . k_j).  Required (not NULL).
 *   B, H, N  batch, heads, sequence length (queries = keys = N); each >= 1.
 *   d        head dimension: 64 or 128 (the method needs whole rows of Q and
 *            K on chip, so d must be small: the Triton article's section on
 *            tiled attention).
 *   scale    multiplier of the scores, finite and > 0 (usually 1/sqrt(d)).
 *   causal   0: every key visible; 1: key j visible to query i iff j <= i.
 *   stream   HIP stream (a hipStream_t passed as void*; NULL = null stream).
 *   dtype    an fa_dtype value.
 *
 * Ownership: all buffers belong to the caller.  The library allocates no
 * device memory and keeps no state between calls, so the extra memory of the
 * operation is L alone, O(N) per row block.  Safe to call from several host
 * threads.
 *
 * Semantics: enqueues one kernel on `stream` and returns once it is enqueued;
 * it does not synchronise.  Results are valid after the stream is
 * synchronised.  Repeated calls on identical inputs give bitwise-identical
 * outputs (no atomics, fixed reduction order).
 *
 * Errors: arguments are checked on the host first; a failed check returns
 * its negative code with nothing enqueued and no HIP call made.  A launch
 * failure returns FA_ERR_HIP.  Faults inside the kernel surface at the
 * caller's next synchronisation, as usual for HIP.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
           int64_t B, int64_t H, int64_t N, int64_t d,
           float scale, int causal, void* stream, int dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
