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
 * Preconditions: B, H, N >= 1; d in {64, 96, 128, 256}; causal in {0, 1};
 *   scale finite and > 0; B*H*N*d < 2^31 elements per tensor and
 *   (N + 256)*d*4 < 2^31 (one head's fp32 slab is addressed with 32-bit
 *   byte offsets).
 * Magnitude limit (not checked): every |v| <= 2^64.  The forward accumulates
 *   P V in fp32 with each P up to 2^40 times the row's current reference
 *   before it renormalises, over up to 2^22 keys, so the accumulators stay
 *   below 2^126 within that limit; larger values can overflow them to
 *   inf/NaN where the exact result is finite.
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
  FA_ERR_HEAD_DIM = -3,  /* d is not 64, 96, 128 or 256 */
  FA_ERR_SCALE = -4,     /* scale not finite or not > 0 */
  FA_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = -6, /* workspace missing or smaller than the matching *_workspace_bytes() */
  FA_ERR_DEVICE = -7,    /* current device is not gfx950, or its properties cannot be read */
  FA_ERR_HIP = -8,       /* a HIP launch or runtime call failed */
  FA_ERR_ARG = -9,       /* causal not 0/1, a part count out of range, or outputs alias inputs */
  FA_ERR_SCRATCH = -10   /* fa_bwd_noalloc: the problem needs more than its 32 MiB of scratch */
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

/*
 * fa_bwd_noalloc - fa_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same parameters, layout, results
 * and kernels as fa_bwd, minus workspace and workspace_bytes; the caller still
 * passes every input and output.  The workspace lives in a file-scope device
 * array of 32 MiB inside libfa.so: each GPU the library runs on holds its own
 * copy from the library's first use on that device until the process ends.
 * The call allocates and frees nothing.  Limit: fa_bwd_workspace_bytes(B, H,
 * N, d) <= 32 MiB (B*H*N up to about 4.19 M rows), else FA_ERR_SCRATCH before
 * anything is enqueued.  Every call on one GPU shares that GPU's array (the
 * kernels overwrite it completely before reading it, so nothing needs
 * clearing): calls that overlap in time on one GPU, on different streams or
 * from different threads, race on it and must be ordered by the caller.
 * The first call on a device looks the array's device address up
 * (hipGetSymbolAddress) and keeps it for that device.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_fwd_fp16, fa_bwd_fp16 - fp16 (IEEE binary16) versions of fa_fwd and
 * fa_bwd with identical parameter lists and conventions: every [B][H][N][d]
 * tensor (q, k, v, o, dO, dq, dk, dv) is _Float16 instead of __bf16, the
 * products run on the fp16 MFMA with fp32 accumulation, and the values
 * rounded to 16 bits (P and dS for the second products, the outputs) are
 * rounded to fp16 (round-to-nearest-even).  lse and the workspace are as in
 * fa_fwd / fa_bwd (fa_bwd_workspace_bytes gives the size).  For the FP16 half
 * of the pages' mixed precision (FlashAttention optimisation page, section
 * 6.2: FP16/BF16 storage with the statistics kept in fp32).
 */
int fa_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, float scale, int causal, hipStream_t stream);
int fa_bwd_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_fwd_dropout, fa_bwd_dropout - bf16 forward and backward with dropout on
 * the attention probabilities (the Journal of Software 2026(1) p.218 survey
 * lists dropout among the operations fused into the kernel, sentence after
 * Eq. (2)).  Parameters as fa_fwd / fa_bwd plus:
 *   dropout_p: drop probability, 0 <= p < 1 (else FA_ERR_ARG); it is applied as
 *     t = round(256 p) clamped to 255 (effective probability t/256), and kept
 *     probabilities are scaled by 1 / (1 - t/256);
 *   seed: 64-bit key of the Philox4x32-10 counter-based generator (Salmon et
 *     al., SC 2011).  Element (b, h, i, j) takes byte j%4 of word i%4 of the
 *     call with counter (i/4, j/4, b*H+h, 0) and key (seed lo, seed hi) and is
 *     kept iff that byte is >= t.  The mask is regenerated, not stored: the
 *     backward must receive the same p, seed, scale and causal as the forward.
 * Forward: o = (P * Z) V with Z = keep / (1 - t/256); lse is the statistic of
 * the softmax before dropout.  Backward: gradients of sum(o * dO) through the
 * same mask; fa_bwd_workspace_bytes gives the workspace size.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed, hipStream_t stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   float dropout_p, unsigned long long seed,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_fwd_splitkv_parts - number of key parts fa_fwd_splitkv uses for these
 * sizes and this num_splits (<= 0: automatic), or 0 if the sizes are
 * invalid.  The keys of every row are cut into ranges of whole 64-key tiles;
 * a request is capped at the number of tiles and at 64, and parts that would
 * hold no tile are dropped.  The automatic choice aims at 512 workgroups of
 * 128 query rows (two per CU), with at least two tiles per part and at most
 * 16 parts; grids that already have 512 workgroups get 1 part.
 */
int fa_fwd_splitkv_parts(int B, int H, int N, int d, int num_splits);

/*
 * fa_fwd_splitkv_workspace_bytes - bytes of workspace fa_fwd_splitkv needs:
 * fp32 partial outputs [S][B][H][N][d] and fp32 partial log-sum-exps
 * [S][B][H][N] for S = fa_fwd_splitkv_parts(...) parts, each rounded up to
 * 256 bytes.  Returns 0 when S is 1 (no workspace needed) or the sizes are
 * invalid.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits);

/*
 * fa_fwd_splitkv - bf16 forward attention with exactly the inputs, outputs
 * and conventions of fa_fwd, computed with the keys of every row split into
 * S = fa_fwd_splitkv_parts(B,H,N,d,num_splits) ranges that separate
 * workgroups process in parallel; each range yields a normalised partial
 * output (fp32) and its log-sum-exp, and the parts are then merged by Eq. (2)
 * of the Journal of Software 2026(1) p.218 survey (as fa_lse_merge does).
 * For grids too small to fill the GPU (few heads, short sequences) this
 * keeps every CU busy.  S == 1 runs fa_fwd's kernel and needs no workspace.
 * workspace: device buffer of at least fa_fwd_splitkv_workspace_bytes(...)
 * bytes (may be NULL when that is 0), owned by the caller, 16-byte aligned,
 * not overlapping any tensor argument; contents on entry do not matter.
 * Results agree with fa_fwd to rounding (the fp32 partials add one more
 * rounding step), not bit for bit.
 * Errors: as fa_fwd, plus FA_ERR_WORKSPACE (missing or too small).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, int num_splits,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_lse_merge - merge S partial attention results over disjoint key sets by
 * Eq. (2) of the Journal of Software 2026(1) p.218 survey: for every row,
 * with M = max_s lse_parts[s] and w_s = e^(lse_parts[s] - M),
 *   o   = sum_s w_s o_parts[s] / sum_s w_s   (fp32, rounded once to bf16),
 *   lse = M + ln sum_s w_s.
 * o_parts: float [S][B][H][N][d], each part normalised by its own sum;
 * lse_parts: float [S][B][H][N], natural-log log-sum-exp of each part (-inf
 * for a row that saw no key in that part: such a part is ignored).  o:
 * __bf16 [B][H][N][d] and lse: float [B][H][N] outputs; a row whose parts
 * are all -inf gets o = 0 and lse = -inf.  S = num_parts in [1, 4096].
 * This is the single-GPU half of attention over keys sharded across devices:
 * each shard's fa_fwd output, converted to fp32, is one part.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEAD_DIM, FA_ERR_ALIGN,
 * FA_ERR_ARG (num_parts out of range or outputs overlapping inputs),
 * FA_ERR_DEVICE, FA_ERR_HIP.
 */
int fa_lse_merge(const float* o_parts, const float* lse_parts, int num_parts, void* o, float* lse,
                 int B, int H, int N, int d, hipStream_t stream);

/*
 * fa_fwd_window - bf16 forward attention restricted to a sliding window:
 * key j is visible to query i iff i - window_left <= j <= i + window_right,
 * where a negative bound means no limit on that side ((-1, -1) is fa_fwd
 * without a mask, (-1, 0) is fa_fwd with causal = 1, (512, 512) is the
 * window of the FlashAttention-2 principle and deployment page's SDPA
 * example).  Every query sees at least itself.  Inputs, outputs (o, lse) and
 * conventions as fa_fwd; key tiles outside every row's window are skipped.
 * Errors: as fa_fwd (without the causal flag).
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int window_left, int window_right,
                  hipStream_t stream);

/*
 * fa_fwd_blocksparse - bf16 forward attention over the kept blocks of a
 * block-sparse mask (block-sparse FlashAttention: FlashAttention
 * optimisation page, section 7).  The N x N score matrix is cut into 64 x 64
 * blocks; block_mask[h][i/64][j/64] != 0 keeps the block containing (i, j),
 * 0 drops it.  block_mask: device pointer to unsigned char
 * [H][nb][nb] (mask_per_head = 1) or [nb][nb] shared by every head
 * (mask_per_head = 0), nb = ceil(N / 64), any alignment, read only.  With
 * causal = 1 the causal mask applies on top.  Dropped blocks cost neither
 * loads nor MFMAs.  A row that sees no key gets o = 0 and lse = -inf.
 * Other inputs, outputs and conventions as fa_fwd.
 * Preconditions beyond fa_fwd's: N <= 65536 (FA_ERR_SHAPE), mask_per_head in
 * {0, 1} (FA_ERR_ARG), block_mask not NULL (FA_ERR_NULL) and not
 * overlapping o or lse (FA_ERR_ARG).
 */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, float scale, int causal,
                       const unsigned char* block_mask, int mask_per_head, hipStream_t stream);

/*
 * fa_bwd_window, fa_bwd_blocksparse - bf16 backward of fa_fwd_window and
 * fa_fwd_blocksparse: the gradients dq, dk, dv of sum(o * dO) for the same
 * visible set, by the recomputation of fa_bwd (FlashAttention-from-GPU-memory
 * page, section 2.2; FlashAttention optimisation page, section 4.2).  o and
 * lse are exactly what the matching forward returned for the same window or
 * mask (a row that saw no key: o = 0, lse = -inf; its dq row is 0 and it adds
 * nothing to dk, dv).  Query steps and key tiles outside every visible block
 * are skipped.  Parameters, layouts, workspace (fa_bwd_workspace_bytes) and
 * ownership as fa_bwd; window_left / window_right as fa_fwd_window;
 * causal, block_mask and mask_per_head as fa_fwd_blocksparse.
 * Errors: as fa_bwd, plus (block-sparse) N <= 65536 (FA_ERR_SHAPE),
 * mask_per_head in {0, 1} (FA_ERR_ARG), block_mask not NULL (FA_ERR_NULL) and
 * not overlapping dq, dk, dv or the workspace (FA_ERR_ARG).
 */
int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                  int window_left, int window_right, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);
int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                       int causal, const unsigned char* block_mask, int mask_per_head, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * fp16 versions of the key split, the merge, the masks and dropout:
 * fa_fwd_splitkv_fp16, fa_lse_merge_fp16, fa_fwd_window_fp16,
 * fa_bwd_window_fp16, fa_fwd_blocksparse_fp16, fa_bwd_blocksparse_fp16,
 * fa_fwd_dropout_fp16, fa_bwd_dropout_fp16.  Each has exactly the parameter
 * list, preconditions, errors and ownership of the entry point without the
 * suffix, with every [B][H][N][d] 16-bit tensor (q, k, v, o, dO, dq, dk, dv)
 * in IEEE binary16 (_Float16) instead of bf16, as fa_fwd_fp16 / fa_bwd_fp16
 * do for fa_fwd / fa_bwd (FlashAttention optimisation page, section 6.2: FP16
 * or BF16 storage).  lse, the fp32 parts of the key split and the workspaces
 * are unchanged (fa_fwd_splitkv_workspace_bytes and fa_bwd_workspace_bytes
 * give their sizes).  P and dS are rounded to fp16 for the MFMAs; the result
 * is rounded once to fp16 (round to nearest even).
 */
int fa_fwd_splitkv_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, float scale, int causal, int num_splits,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_lse_merge_fp16(const float* o_parts, const float* lse_parts, int num_parts, void* o, float* lse,
                      int B, int H, int N, int d, hipStream_t stream);
int fa_fwd_window_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, float scale, int window_left, int window_right,
                       hipStream_t stream);
int fa_bwd_window_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                       int window_left, int window_right, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);
int fa_fwd_blocksparse_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, int d, float scale, int causal,
                            const unsigned char* block_mask, int mask_per_head, hipStream_t stream);
int fa_bwd_blocksparse_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                            int causal, const unsigned char* block_mask, int mask_per_head, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);
int fa_fwd_dropout_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, float scale, int causal, float dropout_p,
                        unsigned long long seed, hipStream_t stream);
int fa_bwd_dropout_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int causal, float dropout_p, unsigned long long seed, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * fa_probe_mfma_bf16 - measurement helper, not part of the attention path:
 * launches `workgroups` workgroups of four waves (two per SIMD), each wave
 * running `iters` rounds of four independent bf16 32x32x16 MFMA accumulation
 * chains on register operands, and writes one float per thread to `sink`
 * (device, >= workgroups*256 floats, 16-byte aligned).  Timing it gives the
 * dense bf16 MFMA rate the GPU sustains, to set beside the published peak:
 * FLOP per call = workgroups * 4 * iters * 4 * 32768.  Errors: FA_ERR_NULL,
 * FA_ERR_ARG (workgroups outside [1, 2^20] or iters < 1), FA_ERR_ALIGN,
 * FA_ERR_DEVICE, FA_ERR_HIP.
 */
int fa_probe_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t stream);

/* fa_status_string - static, human-readable text for a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
