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
  FA_F32 = 1,  /* float32 inputs and output, float32 arithmetic */
  FA_F16 = 2   /* IEEE half inputs and output, float32 accumulation; the
                  exponentials are taken in float32, so the half-precision
                  overflow of e^x past x = 11.09 that the FlashAttention blog
                  post's "(Safe) Softmax" section warns of does not arise */
} fa_dtype;

/* Status codes.  Every negative code except FA_ERR_HIP is returned by the
 * host-side argument checks, before any HIP runtime call is made. */
typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,           /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,          /* B, H or N < 1, or a size too large to index
                                 (bf16, fp16: one head of K, N * d * 2 bytes,
                                 must be below 2^31) */
  FA_ERR_UNSUPPORTED_D = -3,  /* head dimension d is not 32, 64, 128 or 256
                                 (block-sparse and backward: not 32, 64, 128) */
  FA_ERR_DTYPE = -4,          /* dtype is not an fa_dtype value */
  FA_ERR_SCALE = -5,          /* scale is not finite or not > 0 */
  FA_ERR_ALIGN = -6,          /* Q, K, V or O not 16-byte aligned, or L not 4-byte aligned */
  FA_ERR_ALIAS = -7,          /* O or L overlaps an input, or O overlaps L */
  FA_ERR_HIP = -8,            /* the HIP runtime reported an error at launch */
  FA_ERR_ARG = -9,            /* causal is not 0 or 1 */
  FA_ERR_SPLITS = -10,        /* num_splits is not in [1, 128] */
  FA_ERR_WORKSPACE = -11,     /* workspace NULL, too small or not 256-byte aligned */
  FA_ERR_SCRATCH = -12        /* fa_fwd_splitkv_noalloc: the call needs more than
                                 FA_NOALLOC_SCRATCH_BYTES of split workspace */
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
 *            With FA_BF16 or FA_F16, N * d * 2 must be below 2^31
 *            (N < 8388608 at d = 128): K and V are read through 32-bit
 *            buffer offsets.
 *   d        head dimension: 32, 64, 128 or 256 (the method needs whole rows
 *            of Q and K on chip, so d must be small: the Triton article's
 *            section on tiled attention).
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

/*
 * Key-range split forward (for few query blocks per head, where one
 * workgroup per query block leaves most of the chip idle).
 *
 * The query rows are taken in blocks of 256 (rows 256 rb .. 256 rb + 255).
 * The keys visible to block rb -- all N, or with causal = 1 the first
 * V_rb = min(N, 256 (rb + 1)) -- are cut into num_splits ranges on 64-key
 * boundaries: with T_rb = ceil(V_rb / 64) tiles, range s of block rb is
 * keys [64 floor(s T_rb / S), min(V_rb, 64 floor((s+1) T_rb / S))).  Cutting
 * the visible keys rather than all N gives each range of a causal block the
 * same work.  A first kernel computes, for every query row and every range s
 * of its block, the attention of the row over that range alone: its output
 * O_s, already divided by its own softmax denominator, and its logsumexp L_s
 * (-inf, with O_s = 0, when no key of the range is visible to the row).  A
 * second kernel combines the ranges with the softmax-of-a-concatenation rule
 * (the Triton article, section "瓦片注意力计算": m = max(m1, m2),
 * l = e^(m1-m) l1 + e^(m2-m) l2), carried over to O because O is linear in
 * the softmax weights:
 *     L = ln sum_s e^(L_s),     O = sum_s e^(L_s - L) O_s.
 * The result equals fa_fwd's up to float rounding (not bitwise: the sums are
 * grouped differently).
 *
 * fa_fwd_splitkv_workspace returns the workspace size in bytes,
 * num_splits * B*H*N * (d + 1) * 4, or a negative fa_status
 * (FA_ERR_SHAPE, FA_ERR_UNSUPPORTED_D, FA_ERR_SPLITS).  It makes no HIP call.
 *
 * fa_fwd_splitkv takes fa_fwd's arguments plus
 *   num_splits       number of key ranges, 1..128; ranges beyond the number
 *                    of key tiles are empty and cost one idle workgroup each.
 *   workspace        device pointer, 256-byte aligned, owned by the caller,
 *                    at least fa_fwd_splitkv_workspace(...) bytes, not
 *                    overlapping Q, K, V, O or L.  Overwritten: float32
 *                    O_s [num_splits][B*H*N][d] followed by float32
 *                    L_s [num_splits][B*H*N].  Its contents after the call are
 *                    these partials; nothing needs to be cleared before.
 *   workspace_bytes  size of the workspace buffer.
 * It enqueues the two kernels on `stream` and does not synchronise.  The
 * checks and errors are fa_fwd's, plus FA_ERR_SPLITS and FA_ERR_WORKSPACE;
 * FA_ERR_ALIAS also covers a workspace overlapping another buffer.  Two calls
 * that share one workspace must be ordered (same stream or an event).
 * Deterministic: identical inputs give bitwise-identical outputs.
 */
int64_t fa_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t d, int num_splits);

int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* L,
                   int64_t B, int64_t H, int64_t N, int64_t d,
                   float scale, int causal, void* stream, int dtype,
                   int num_splits, void* workspace, int64_t workspace_bytes);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, result and errors are fa_fwd_splitkv's without `workspace` and
 * `workspace_bytes`.  The partials go to a scratch buffer inside the library
 * (a static device array of FA_NOALLOC_SCRATCH_BYTES, one per device, held
 * until the process ends); the call allocates and frees nothing.  A call
 * needing more than FA_NOALLOC_SCRATCH_BYTES, i.e.
 * fa_fwd_splitkv_workspace(B, H, N, d, num_splits) > FA_NOALLOC_SCRATCH_BYTES,
 * returns FA_ERR_SCRATCH before any HIP call.  Every element of the scratch
 * that a call reads it has written first, so nothing is cleared and the
 * contents left by an earlier call do not matter.
 *
 * All calls on one device share that device's buffer: two calls that may run
 * at the same time on one device (different streams without ordering) race
 * on it and give undefined results.  Order them (one stream, or events).
 */
#define FA_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

int fa_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* L,
                           int64_t B, int64_t H, int64_t N, int64_t d,
                           float scale, int causal, void* stream, int dtype,
                           int num_splits);

/*
 * fa_fwd_blocksparse -- fa_fwd restricted to the key blocks a block mask
 * enables (the block-sparse attention kernel announced in the introduction
 * of the Triton article "理解 Flash Attention：在 Triton 中从头编写算法").
 *
 *   block_mask  device pointer, uint8 [mask_heads][nb][nb], nb = ceil(N/64),
 *               row-major, owned by the caller, read only.  Byte [m][i][j]
 *               nonzero: the queries of 64-row block i may see the keys of
 *               64-key block j (the last block of each side may be partial).
 *   mask_heads  1 (one mask for every head), H (mask h for head h of every
 *               batch) or B*H (mask b*H + h).
 *
 * Key j is visible to query i iff block_mask[m][i/64][j/64] != 0 and, with
 * causal = 1, j <= i.  Hidden scores are -inf before the softmax, so the
 * result is the definition under that mask; a row with no visible key gets
 * O = 0 and L = -inf.  Only key blocks that some query block of a
 * workgroup sees are loaded and multiplied.  The other arguments, the
 * ownership and the semantics are fa_fwd's.
 *
 * Errors: fa_fwd's checks, plus FA_ERR_NULL for a NULL mask, FA_ERR_ARG for
 * another mask_heads, FA_ERR_ALIAS if the mask overlaps O or L, and
 * FA_ERR_SHAPE when the per-workgroup list of key blocks (4 bytes per key
 * block, held on chip next to the K and V buffers) does not fit: with bf16,
 * N up to about 1,048,000 at d = 128.
 */
int fa_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* L,
                       int64_t B, int64_t H, int64_t N, int64_t d,
                       float scale, int causal, void* stream, int dtype,
                       const uint8_t* block_mask, int64_t mask_heads);

/*
 * fa_bwd -- gradients of a scalar loss through O = softmax(scale Q K^T
 * [+ causal mask]) V: given dO = dLoss/dO, returns dQ, dK and dV.  The score
 * matrix is recomputed from Q, K and the forward's logsumexp L rather than
 * stored (the recomputation of the Triton article "理解 Flash Attention：在
 * Triton 中从头编写算法", section "核心思想").  With P = exp(scale S - L):
 *     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_d dO_id O_id,
 *     dQ = scale dS K,  dK = scale dS^T Q.
 *
 *   Q, K, V   the forward's inputs, [B, H, N, d], element type `dtype`.
 *   O, L      the forward's outputs for the same inputs, scale and causal
 *             (fa_fwd's O and L).  Read only.
 *   dO        device pointer, [B, H, N, d], element type `dtype`.  Read only.
 *   dQ, dK, dV  device pointers, [B, H, N, d], element type `dtype`.  Written.
 *   B, H, N, d, scale, causal, stream, dtype   as for fa_fwd; d is 32, 64 or
 *             128 (FA_ERR_UNSUPPORTED_D otherwise).
 *   workspace        device pointer, 256-byte aligned, owned by the caller,
 *                    at least fa_bwd_workspace(...) bytes (float32 D, one per
 *                    row), overwritten; nothing needs clearing before.
 *   workspace_bytes  size of the workspace buffer.
 * fa_bwd_workspace returns that size in bytes (4 * B * H * N), or a negative
 * fa_status (FA_ERR_SHAPE, FA_ERR_UNSUPPORTED_D) for arguments fa_bwd rejects;
 * FA_ERR_SHAPE also when 4 * B * H * N does not fit a signed 64-bit size.
 *
 * Every buffer lives in device memory of the current device and stays owned
 * by the caller.  Three kernels are enqueued on `stream` (D, then dK and dV,
 * then dQ); the call does not synchronise.  No result is accumulated across
 * workgroups, so identical inputs give bitwise-identical gradients.
 *
 * Errors: fa_fwd's checks (with O and L in the place of fa_fwd's outputs),
 * FA_ERR_NULL for a NULL dO, dQ, dK or dV, FA_ERR_ALIGN if one of them is not
 * 16-byte aligned, FA_ERR_WORKSPACE, and FA_ERR_ALIAS if any written buffer
 * (dQ, dK, dV, workspace) overlaps another buffer.
 */
int64_t fa_bwd_workspace(int64_t B, int64_t H, int64_t N, int64_t d);

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* L, void* dQ, void* dK, void* dV,
           int64_t B, int64_t H, int64_t N, int64_t d,
           float scale, int causal, void* stream, int dtype,
           void* workspace, int64_t workspace_bytes);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
