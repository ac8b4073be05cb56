/*
 * flash_attn.h -- C interface of libflashattn.so: exact scaled dot-product
 * attention on an AMD Instinct MI355X (gfx950) -- the fused forward pass
 * (non-causal and causal), its gradients, and a three-pass comparator.
 *
 * The operation (forward entry points; the causal form restricts row i to
 * keys 0..i, see flash_attn_fwd_causal):
 *   for every batch b and head h, with S = scale * Q K^T over the N tokens,
 *     O   = softmax_rows(S) V
 *     LSE = ln sum_j exp(S_ij)                 (natural log, one per query row)
 *   This is attention as defined in "FlashAttention" (interactiveprimer),
 *   intro and "The bottleneck is memory, not multiplication": an N x N score
 *   matrix, a row softmax, a product with the values. "scale" is the caller's
 *   factor (the pages say the scores are scaled but fix no value; 1/sqrt(d)
 *   is the usual choice). LSE is the softmax's per-row normaliser ln(sum);
 *   it is not on the pages and is returned so partial results can be merged.
 *
 * Layout (all entry points):
 *   q, k, v, o : contiguous [B, H, N, d] of the element type `dtype`, row major,
 *                d fastest. o has the element type of the inputs.
 *   lse        : contiguous [B, H, N] float32.
 *   Every pointer is a DEVICE pointer owned by the caller; the library keeps
 *   none of them after a call returns. Outputs must not alias inputs.
 *   Base pointers must be 16-byte aligned.
 *
 * Supported: dtype FA_F32, FA_F16, FA_BF16; d in {64, 128}; any N >= 1.
 * B, H or N equal to 0 is an empty problem: FA_OK, nothing is launched or
 * written, and pointers are not examined.
 *
 * Errors: arguments are validated before any HIP call; on a validation error
 * nothing is launched and nothing is written. FA_ERR_HIP reports a launch
 * failure (hipGetLastError after the launch). NaN or Inf inputs are not
 * screened: they propagate into the outputs.
 *
 * Streams: `stream` is a hipStream_t passed as void*; NULL selects the null
 * stream. Kernels are launched on the calling thread's current HIP device,
 * and `stream` must belong to that device. Calls are asynchronous on that
 * stream and never synchronise. The library holds no per-call state (only
 * per-device caches of the compute-unit count and of the address of
 * flash_attn_bwd_noalloc's fixed scratch, each filled on first use), so calls
 * from several host threads are safe, except overlapping calls of
 * flash_attn_bwd_noalloc on one device (see there).
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  FA_ERR_SHAPE = 2,       /* a negative size, or a size product overflows   */
  FA_ERR_UNSUPPORTED = 3, /* unsupported dtype or head size d               */
  FA_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned          */
  FA_ERR_WORKSPACE = 5,   /* naive path: workspace smaller than one head    */
  FA_ERR_SCALE = 6,       /* scale is NaN or infinite                       */
  FA_ERR_HIP = 7,         /* the HIP runtime reported an error at launch    */
  FA_ERR_TOO_LARGE = 8    /* flash_attn_bwd_noalloc: B*H*N > FA_NOALLOC_MAX_ROWS */
} fa_status;

/*
 * flash_attn_fwd -- the fused, tiled forward pass.
 *
 * Method: "FlashAttention, simplified", section "The trick", and
 * "FlashAttention" (interactiveprimer), "The bottleneck is memory, not
 * multiplication": one workgroup per (batch, head, tile of query rows) keeps
 * its query tile on chip, streams K and V tiles through on-chip memory, keeps
 * a running row maximum and running sum (online softmax), rescales its
 * accumulator when the maximum grows and divides by the sum once at the end.
 * The N x N scores never reach device memory; device-memory traffic is
 * O(N) per head ("What FlashAttention actually buys", "The actual problem").
 *
 * Arguments: q, k, v [B,H,N,d] inputs; o [B,H,N,d] output; lse [B,H,N] float32
 * output, or NULL to skip it; scale finite (any sign; 0 gives the mean of V).
 * Arithmetic: for FA_F16/FA_BF16, products on the matrix cores with float32
 * accumulation, softmax statistics in float32, probabilities rounded to the
 * input type before the product with V, O rounded to nearest even. For
 * FA_F32 every step is float32.
 * Results are deterministic: the same inputs give bitwise the same outputs.
 * Returns an fa_status.
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * flash_attn_fwd_causal -- the fused forward pass with causal (prefill)
 * masking: query i of a sequence attends keys 0..i only, i.e. row i's softmax
 * and LSE run over S_i0 .. S_ii. The pages name the prefill case
 * ("FlashAttention, simplified", "Why it matters for inference") but no mask;
 * this is the lower-triangular reading, with queries and keys indexed from
 * the same first token (N queries, N keys).
 * Arguments, layout, arithmetic, determinism and errors as flash_attn_fwd.
 * Key tiles entirely after a query tile are skipped, so the work is about
 * half that of flash_attn_fwd.
 */
int flash_attn_fwd_causal(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * flash_attn_bwd -- gradients of flash_attn_fwd: given the forward's inputs
 * q, k, v, its outputs o and lse, and the upstream gradient dout = dL/dO,
 * writes dq = dL/dQ, dk = dL/dK, dv = dL/dV. With P = exp(scale Q K^T - LSE):
 *   dV = P^T dO,  dS = P * (dO V^T - D),  D_i = dO_i . O_i,
 *   dQ = scale dS K,  dK = scale dS^T Q.
 * The score tiles are recomputed from lse rather than stored ("What
 * FlashAttention actually buys", "Why the distinction matters downstream"):
 * nothing N x N is written.
 *
 * Arguments: q, k, v, o, dout, dq, dk, dv: [B,H,N,d] device pointers of
 * `dtype` (FA_F32, FA_F16 or FA_BF16); lse: the
 * [B,H,N] float32 output of the forward pass with the same inputs and scale;
 * delta: caller-owned float32 scratch of 2*B*H*N elements, overwritten with
 * D ([B,H,N], first half) and LSE*log2(e) ([B,H,N], second half); the
 * library allocates nothing. All 16-byte aligned; outputs must not alias
 * inputs. Three kernels run in order on `stream`. Arithmetic: products on the
 * matrix cores with float32 accumulation; for FA_F16/FA_BF16, P and dS are
 * rounded to the input type before their products and the gradients to
 * nearest even; for FA_F32 every step is float32. Deterministic (no
 * atomics). Validation and status codes as flash_attn_fwd (d in {64,128}).
 */
int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, float* delta,
                   int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * flash_attn_bwd_causal -- the gradients of flash_attn_fwd_causal (query i
 * attends keys 0..i); lse must come from flash_attn_fwd_causal. Arguments as
 * flash_attn_bwd.
 */
int flash_attn_bwd_causal(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* delta,
                          int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * flash_attn_bwd_noalloc -- flash_attn_bwd without the caller's `delta`
 * scratch, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation). The
 * library keeps the 2*B*H*N floats of row statistics in a fixed device array
 * of FA_NOALLOC_MAX_ROWS * 2 floats (32 MiB), one per device, held from the
 * library's load until the process ends; the call allocates and frees nothing.
 * Its device address is looked up on the first call on each device.
 *
 * Arguments, layout, arithmetic, results and status codes as flash_attn_bwd
 * (non-causal), minus `delta`; gradients are bitwise those of flash_attn_bwd.
 * B*H*N above FA_NOALLOC_MAX_ROWS returns FA_ERR_TOO_LARGE before any HIP
 * call. Every call on one device shares that device's array and overwrites it
 * before reading it: calls that overlap on one device (on different streams,
 * or from several host threads without ordering) race and may return wrong
 * gradients. Calls ordered on one stream are safe.
 */
#define FA_NOALLOC_MAX_ROWS 4194304
int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv,
                           int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * attn_naive_workspace_bytes -- workspace for attn_naive_fwd to process every
 * head in one pass: B*H*N*N*(4 + e) bytes, e = element size of dtype (S is
 * held in float32, P in the input type). Any workspace of at least one head,
 * N*N*(4 + e) bytes, is accepted: heads are then processed in chunks.
 * Returns 0 for an unsupported dtype, a negative size or on overflow.
 */
size_t attn_naive_workspace_bytes(int B, int H, int N, int dtype);

/*
 * attn_naive_fwd -- standard, materialising attention in three passes, kept
 * as the traffic comparator ("FlashAttention, simplified", "The problem";
 * "What FlashAttention actually buys", "The actual problem"):
 *   pass 1  S = scale * Q K^T            written to the workspace (float32)
 *   pass 2  P = softmax_rows(S), LSE     S read back, P written (input type)
 *   pass 3  O = P V                      P read back
 * Same arguments, layout and result as flash_attn_fwd, plus `workspace`, a
 * caller-owned device buffer of `workspace_bytes` (16-byte aligned), which is
 * overwritten. Fails with FA_ERR_WORKSPACE if it holds less than one head.
 * lse may be NULL.
 */
int attn_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/* fa_strerror -- a static, human-readable string for an fa_status value. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
