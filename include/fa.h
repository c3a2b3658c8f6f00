/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The operation: exact scaled-dot-product attention O = softmax(scale*Q K^T) V
 * of the FlashAttention optimisation page (intelliparadigm.com, section 1,
 * steps 1-4), computed tile by tile with the online softmax of the Journal of
 * Software 2026(1) p.218 LLM pre-training survey (Eq. (1) for one block,
 * Eq. (2) for merging two blocks), so the N x N score matrix never reaches
 * HBM.  The problem statement of that survey fixes the data flow: Q, K, V of
 * N rows and d columns live in HBM, the kernel reads them and writes O back.
 * The forward also writes the per-row statistic kept for the backward pass
 * (FlashAttention optimisation page, section 4.1), and the backward pass
 * recomputes P from it (FlashAttention-from-GPU-memory page (jsqmd.com),
 * section 2.2; FlashAttention optimisation page, section 4.2).
 *
 * Common conventions for every entry point
 * ----------------------------------------
 * Layout: every tensor argument is contiguous [B][H][N][d] (row-major, d
 *   fastest); the statistic `lse` is contiguous [B][H][N] float.  Offsets are
 *   computed in 64-bit.
 * Pointers: device pointers on the HIP device that is current when the call
 *   is made, 16-byte aligned.  Outputs must not alias inputs or each other.
 * Ownership: the caller allocates and frees every buffer (the backward
 *   workspace included).  The library allocates no device memory, keeps no
 *   mutable global state, never synchronises and never prints; calls are
 *   re-entrant and thread-safe.
 * Preconditions: B, H, N >= 1; d in {64, 128}; causal in {0, 1};
 *   scale finite and > 0; B*H*N*d < 2^31 elements per tensor and
 *   (N + 256)*d*4 < 2^31 (one head's fp32 slab is addressed with 32-bit
 *   byte offsets).
 * Causal mask: key j is visible to query i iff j <= i (queries and keys have
 *   the same length N).
 * Log-sum-exp: lse[b][h][i] = ln( sum over visible j of exp(scale * q_i . k_j) ),
 *   natural logarithm.
 * Errors: every check runs before anything is enqueued; on error the call
 *   returns a negative fa_status and writes nothing.  A device that is not
 *   gfx950 gives FA_ERR_DEVICE; a failed launch gives FA_ERR_HIP.
 * Asynchrony: work is enqueued on `stream` (0 = the null stream) in stream
 *   order; results are valid once the caller has synchronised that stream.
 *   Faults inside a kernel surface at the caller's next synchronisation.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,     /* B, H or N < 1, or a tensor or head too large for 32-bit offsets */
  FA_ERR_HEAD_DIM = -3,  /* d is not 64 or 128 */
  FA_ERR_SCALE = -4,     /* scale not finite or not > 0 */
  FA_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = -6, /* backward workspace missing or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_DEVICE = -7,    /* current device is not gfx950, or its properties cannot be read */
  FA_ERR_HIP = -8,       /* a HIP launch or runtime call failed */
  FA_ERR_ARG = -9        /* causal not 0/1, or outputs alias inputs */
} fa_status;

/*
 * fa_fwd - bf16 forward attention.
 * q, k, v: __bf16 [B][H][N][d] inputs.  o: __bf16 [B][H][N][d] output, each
 * row normalised in fp32 and rounded once (round-to-nearest-even).
 * lse: float [B][H][N] output, natural-log log-sum-exp of each score row.
 * Products QK^T and PV run in bf16 with fp32 accumulation; the probabilities
 * fed to PV are rounded to bf16, the softmax statistics stay fp32.
 * Defined by: FlashAttention optimisation page, section 4.1 (forward steps);
 * FlashAttention-2 principle and deployment page (yunthe.com), tiled code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_fwd_f32 - fp32 forward attention with the same parameter meaning as
 * fa_fwd; every tensor (q, k, v, o) is float [B][H][N][d] and nothing is
 * rounded below fp32.  For callers that need results that agree with the
 * plain definition to float32 accuracy (FlashAttention-2 principle and
 * deployment page, troubleshooting item 2: compute in float32 to match).
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_bwd_workspace_bytes - size in bytes of the workspace fa_bwd needs for
 * these sizes: the fp32 row terms D = rowsum(dO * O) [B][H][N] and the fp32
 * LSE in base-2 units [B][H][N] (each padded to 256 bytes).  Returns 0 if
 * the sizes are invalid.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd - bf16 backward attention by recomputation.
 * q, k, v, o: __bf16 [B][H][N][d] (o and lse exactly as fa_fwd returned them
 * for the same q, k, v, scale and causal).  dO: __bf16 [B][H][N][d] gradient
 * of the loss with respect to O.  dq, dk, dv: __bf16 [B][H][N][d] outputs.
 * workspace: device buffer of at least fa_bwd_workspace_bytes(B,H,N,d) bytes,
 * owned by the caller; its contents on entry do not matter and are
 * clobbered.  P is recomputed tile by tile from q, k and lse; the N x N
 * matrices are never written to memory.  dK and dV are accumulated in a
 * key-block-major pass and dQ in a query-block-major pass, both in fp32 on
 * chip without atomics, so the results are bitwise reproducible.
 * Defined by: FlashAttention-from-GPU-memory page, section 2.2
 * (recomputation); FlashAttention optimisation page, section 4.2 (backward
 * tiled like the forward); the gradients are the chain rule on the forward.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fa_status_string - static, human-readable text for a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
