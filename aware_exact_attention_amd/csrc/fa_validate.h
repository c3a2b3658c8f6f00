// fa_validate.h - argument checks of the C ABI, pure C++ (no HIP), so that the
// same code is unit-tested on a CPU-only host with g++ and used by libfa.so.
// Every check runs before anything is enqueued; the first failing check
// decides the status.
#ifndef FA_VALIDATE_H_
#define FA_VALIDATE_H_

#include <cmath>
#include <cstddef>
#include <cstdint>

namespace fa {

// Status values mirror fa_status in include/fa.h.
enum : int {
  kOk = 0, kErrNull = -1, kErrShape = -2, kErrHeadDim = -3, kErrScale = -4,
  kErrAlign = -5, kErrWorkspace = -6, kErrDevice = -7, kErrHip = -8, kErrArg = -9,
  kErrScratch = -10
};

struct Shape {
  int B, H, N, d;
};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Elements per [B][H][N][d] tensor, or -1 if the shape is invalid / too large.
// Besides the 2^31 elements per tensor, one head's fp32 slab plus 256 rows of
// slack must stay below 2^31 bytes: the kernels address a head with 32-bit
// byte offsets, including rows just past N that the buffer bounds discard.
inline int64_t tensor_elems(const Shape& s) {
  if (s.B < 1 || s.H < 1 || s.N < 1 || s.d < 1) return -1;
  const int64_t n = int64_t(s.B) * s.H * s.N * s.d;
  if (n >= (int64_t(1) << 31)) return -1;
  if ((int64_t(s.N) + 256) * s.d * 4 >= (int64_t(1) << 31)) return -1;
  return n;
}

// Head dimensions: 64, 96, 128 and 256 on every entry point.
inline bool head_dim_ok(int d) { return d == 64 || d == 96 || d == 128 || d == 256; }

inline int check_common(const Shape& s, float scale, int causal) {
  if (tensor_elems(s) < 0) return kErrShape;
  if (!head_dim_ok(s.d)) return kErrHeadDim;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return kErrScale;
  if (causal != 0 && causal != 1) return kErrArg;
  return kOk;
}

// Byte ranges [p, p+n) overlap?
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Forward: inputs q,k,v (elem_bytes each element), outputs o (same), lse (float per row).
inline int validate_fwd(const void* q, const void* k, const void* v, const void* o, const void* lse,
                        const Shape& s, float scale, int causal, size_t elem_bytes) {
  if (!q || !k || !v || !o || !lse) return kErrNull;
  int st = check_common(s, scale, causal);
  if (st != kOk) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return kErrAlign;
  const size_t tb = size_t(tensor_elems(s)) * elem_bytes;
  const size_t lb = size_t(s.B) * s.H * s.N * sizeof(float);
  const void* ins[3] = {q, k, v};
  for (const void* in : ins) {
    if (overlaps(in, tb, o, tb) || overlaps(in, tb, lse, lb)) return kErrArg;
  }
  if (overlaps(o, tb, lse, lb)) return kErrArg;
  return kOk;
}

// Workspace of the backward, in this order, each part rounded up to 256
// bytes: the fp32 row terms D = rowsum(dO * O) [B][H][N] and the fp32 LSE in
// base-2 units [B][H][N].
struct BwdWorkspace {
  size_t d, lse2, total;
};

inline BwdWorkspace bwd_workspace_layout(const Shape& s) {
  const int64_t n = tensor_elems(s);
  if (n < 0 || !head_dim_ok(s.d)) return BwdWorkspace{0, 0, 0};
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = size_t(s.B) * s.H * s.N;
  BwdWorkspace w;
  w.d = 0;
  w.lse2 = up(rows * 4);
  w.total = w.lse2 + up(rows * 4);
  return w;
}

inline size_t bwd_workspace_bytes(const Shape& s) { return bwd_workspace_layout(s).total; }

inline int validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* lse,
                        const void* dO, const void* dq, const void* dk, const void* dv,
                        const Shape& s, float scale, int causal,
                        const void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return kErrNull;
  int st = check_common(s, scale, causal);
  if (st != kOk) return st;
  const void* all[9] = {q, k, v, o, lse, dO, dq, dk, dv};
  for (const void* p : all)
    if (!aligned16(p)) return kErrAlign;
  const size_t need = bwd_workspace_bytes(s);
  if (!ws || ws_bytes < need) return kErrWorkspace;
  if (!aligned16(ws)) return kErrAlign;
  const size_t tb = size_t(tensor_elems(s)) * 2;
  const size_t lb = size_t(s.B) * s.H * s.N * sizeof(float);
  const void* ins[6] = {q, k, v, o, lse, dO};
  const size_t insz[6] = {tb, tb, tb, tb, lb, tb};
  const void* outs[4] = {dq, dk, dv, ws};
  const size_t outsz[4] = {tb, tb, tb, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return kErrArg;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return kErrArg;
  }
  return kOk;
}

// ---------------------------------------------------------------------------
// Key-split forward and the merge of parts
// ---------------------------------------------------------------------------
// The split forward runs four-wave workgroups of 128 query rows over 64-key
// tiles; a part is a range of whole tiles.
constexpr int kSplitKeyTile = 64;
constexpr int kSplitRowBlock = 128;
constexpr int kMaxSplits = 64;
// Automatic choice: enough parts for two four-wave workgroups on each of the
// 256 CUs, at least two tiles per part, at most 16 parts.
constexpr long long kSplitTargetWorkgroups = 512;
constexpr int kMaxAutoSplits = 16;
constexpr int kMaxMergeParts = 4096;

// Number of key parts fa_fwd_splitkv uses for `requested` (<= 0: automatic),
// or 0 if the shape is invalid.  Parts that would hold no tile are dropped.
inline int split_count(const Shape& s, int requested) {
  if (tensor_elems(s) < 0 || !head_dim_ok(s.d)) return 0;
  const int tc = (s.N + kSplitKeyTile - 1) / kSplitKeyTile;
  long long S;
  if (requested > 0) {
    S = requested;
  } else {
    const long long g = (long long)s.B * s.H * ((s.N + kSplitRowBlock - 1) / kSplitRowBlock);
    S = g >= kSplitTargetWorkgroups ? 1 : (kSplitTargetWorkgroups + g - 1) / g;
    const long long two_tiles = tc / 2 > 0 ? tc / 2 : 1;
    if (S > two_tiles) S = two_tiles;
    if (S > kMaxAutoSplits) S = kMaxAutoSplits;
  }
  if (S > tc) S = tc;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  const long long tps = (tc + S - 1) / S;
  return int((tc + tps - 1) / tps);
}

// Workspace of the split forward with S > 1 parts, each part rounded up to
// 256 bytes: fp32 partial outputs [S][B][H][N][d], then fp32 partial
// log-sum-exps [S][B][H][N].  S <= 1 needs none.
struct SplitLayout {
  size_t o_parts, lse_parts, total;
};

inline SplitLayout split_workspace_layout(const Shape& s, int S) {
  if (S <= 1 || tensor_elems(s) < 0) return SplitLayout{0, 0, 0};
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = size_t(s.B) * s.H * s.N;
  SplitLayout w;
  w.o_parts = 0;
  w.lse_parts = up(size_t(S) * rows * s.d * 4);
  w.total = w.lse_parts + up(size_t(S) * rows * 4);
  return w;
}

inline size_t split_workspace_bytes(const Shape& s, int requested) {
  return split_workspace_layout(s, split_count(s, requested)).total;
}

inline int validate_fwd_splitkv(const void* q, const void* k, const void* v, const void* o, const void* lse,
                                const Shape& s, float scale, int causal, int requested, const void* ws,
                                size_t ws_bytes) {
  int st = validate_fwd(q, k, v, o, lse, s, scale, causal, 2);
  if (st != kOk) return st;
  const int S = split_count(s, requested);
  if (S > 1) {
    const size_t need = split_workspace_layout(s, S).total;
    if (!ws || ws_bytes < need) return kErrWorkspace;
    if (!aligned16(ws)) return kErrAlign;
    const size_t tb = size_t(tensor_elems(s)) * 2;
    const size_t lb = size_t(s.B) * s.H * s.N * sizeof(float);
    const void* all[5] = {q, k, v, o, lse};
    const size_t sz[5] = {tb, tb, tb, tb, lb};
    for (int i = 0; i < 5; ++i)
      if (overlaps(ws, need, all[i], sz[i])) return kErrArg;
  }
  return kOk;
}

// Merge: o_parts float [S][B][H][N][d], lse_parts float [S][B][H][N] in;
// o bf16 [B][H][N][d], lse float [B][H][N] out.
inline int validate_lse_merge(const void* o_parts, const void* lse_parts, int S, const void* o, const void* lse,
                              const Shape& s) {
  if (!o_parts || !lse_parts || !o || !lse) return kErrNull;
  if (tensor_elems(s) < 0) return kErrShape;
  if (!head_dim_ok(s.d)) return kErrHeadDim;
  if (S < 1 || S > kMaxMergeParts) return kErrArg;
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse)) return kErrAlign;
  const size_t rows = size_t(s.B) * s.H * s.N;
  const size_t ob = rows * s.d * 2, lb = rows * 4;
  const size_t opb = size_t(S) * rows * s.d * 4, lpb = size_t(S) * rows * 4;
  if (overlaps(o, ob, o_parts, opb) || overlaps(o, ob, lse_parts, lpb) || overlaps(lse, lb, o_parts, opb) ||
      overlaps(lse, lb, lse_parts, lpb) || overlaps(o, ob, lse, lb))
    return kErrArg;
  return kOk;
}

// ---------------------------------------------------------------------------
// Tile-skipping masks
// ---------------------------------------------------------------------------
constexpr int kMaskBlockRows = 64;        // block-sparse masks are over 64 x 64 blocks
constexpr int kMaxBlockSparseN = 65536;   // the kernel lists at most 1024 key blocks per row block

inline int validate_fwd_window(const void* q, const void* k, const void* v, const void* o, const void* lse,
                               const Shape& s, float scale) {
  return validate_fwd(q, k, v, o, lse, s, scale, 0, 2);
}

// Bytes of the block mask: [H][nb][nb] (per_head) or [nb][nb], nb = ceil(N/64).
inline size_t block_mask_bytes(const Shape& s, int per_head) {
  const size_t nb = size_t(s.N + kMaskBlockRows - 1) / kMaskBlockRows;
  return (per_head ? size_t(s.H) : 1) * nb * nb;
}

inline int validate_fwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* lse,
                                    const Shape& s, float scale, int causal, const void* block_mask,
                                    int per_head) {
  if (!block_mask || !q || !k || !v || !o || !lse) return kErrNull;
  int st = check_common(s, scale, causal);
  if (st != kOk) return st;
  if (s.N > kMaxBlockSparseN) return kErrShape;
  if (per_head != 0 && per_head != 1) return kErrArg;
  st = validate_fwd(q, k, v, o, lse, s, scale, causal, 2);
  if (st != kOk) return st;
  const size_t mb = block_mask_bytes(s, per_head);
  const size_t tb = size_t(tensor_elems(s)) * 2;
  const size_t lb = size_t(s.B) * s.H * s.N * sizeof(float);
  if (overlaps(block_mask, mb, o, tb) || overlaps(block_mask, mb, lse, lb)) return kErrArg;
  return kOk;
}

// Dropout probability: finite, 0 <= p < 1.
// The masked backward: fa_bwd's preconditions (without the causal flag for
// the window) plus, for a block mask, those of fa_fwd_blocksparse on the mask
// and no overlap of the mask with dq, dk, dv or the workspace.
inline int validate_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* lse,
                               const void* dO, const void* dq, const void* dk, const void* dv, const Shape& s,
                               float scale, const void* ws, size_t ws_bytes) {
  return validate_bwd(q, k, v, o, lse, dO, dq, dk, dv, s, scale, 0, ws, ws_bytes);
}

inline int validate_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* lse,
                                    const void* dO, const void* dq, const void* dk, const void* dv, const Shape& s,
                                    float scale, int causal, const void* block_mask, int per_head, const void* ws,
                                    size_t ws_bytes) {
  if (!block_mask) return kErrNull;
  int st = validate_bwd(q, k, v, o, lse, dO, dq, dk, dv, s, scale, causal, ws, ws_bytes);
  if (st != kOk) return st;
  if (s.N > kMaxBlockSparseN) return kErrShape;
  if (per_head != 0 && per_head != 1) return kErrArg;
  const size_t mb = block_mask_bytes(s, per_head);
  const size_t tb = size_t(tensor_elems(s)) * 2;
  const void* outs[4] = {dq, dk, dv, ws};
  const size_t outsz[4] = {tb, tb, tb, bwd_workspace_bytes(s)};
  for (int i = 0; i < 4; ++i)
    if (overlaps(block_mask, mb, outs[i], outsz[i])) return kErrArg;
  return kOk;
}

// Scratch that the allocation-free backward (fa_bwd_noalloc) keeps in a
// file-scope device array, one per GPU: the backward workspace of every call
// must fit in it.  32 MiB holds the row terms of B*H*N up to about 4.19 M rows.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

// fa_bwd_noalloc: fa_bwd's checks without a caller workspace, plus the
// scratch limit.
inline int validate_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* lse,
                                const void* dO, const void* dq, const void* dk, const void* dv,
                                const Shape& s, float scale, int causal) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return kErrNull;
  int st = check_common(s, scale, causal);
  if (st != kOk) return st;
  const void* all[9] = {q, k, v, o, lse, dO, dq, dk, dv};
  for (const void* p : all)
    if (!aligned16(p)) return kErrAlign;
  if (bwd_workspace_bytes(s) > kNoAllocScratchBytes) return kErrScratch;
  const size_t tb = size_t(tensor_elems(s)) * 2;
  const size_t lb = size_t(s.B) * s.H * s.N * sizeof(float);
  const void* ins[6] = {q, k, v, o, lse, dO};
  const size_t insz[6] = {tb, tb, tb, tb, lb, tb};
  const void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], tb, ins[j], insz[j])) return kErrArg;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], tb, outs[j], tb)) return kErrArg;
  }
  return kOk;
}

inline int check_dropout_p(float p) { return (std::isfinite(p) && p >= 0.0f && p < 1.0f) ? kOk : kErrArg; }

inline const char* status_string(int st) {
  switch (st) {
    case kOk: return "FA_OK: success";
    case kErrNull: return "FA_ERR_NULL: a required pointer is NULL";
    case kErrShape: return "FA_ERR_SHAPE: B, H and N must be >= 1, each tensor < 2^31 elements and (N+256)*d*4 < 2^31";
    case kErrHeadDim: return "FA_ERR_HEAD_DIM: head dimension d must be 64, 96, 128 or 256";
    case kErrScale: return "FA_ERR_SCALE: scale must be finite and > 0";
    case kErrAlign: return "FA_ERR_ALIGN: every pointer must be 16-byte aligned";
    case kErrWorkspace: return "FA_ERR_WORKSPACE: workspace missing or smaller than the *_workspace_bytes() size";
    case kErrDevice: return "FA_ERR_DEVICE: the current device is not a gfx950 GPU";
    case kErrHip: return "FA_ERR_HIP: a HIP launch or runtime call failed";
    case kErrArg: return "FA_ERR_ARG: causal must be 0 or 1, counts and probabilities in range, and outputs must not alias inputs";
    case kErrScratch: return "FA_ERR_SCRATCH: fa_bwd_noalloc needs fa_bwd_workspace_bytes() <= 32 MiB (B*H*N up to about 4.19 M rows)";
    default: return "unknown fa_status";
  }
}

}  // namespace fa

#endif  // FA_VALIDATE_H_
