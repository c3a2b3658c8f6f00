// fa_api.cpp - extern "C" entry points of libfa.so (declared in include/fa.h).
// Validates every argument before anything is enqueued, checks that the
// current device is a gfx950, and launches the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/fa.h"
#include "fa_validate.h"

namespace fa {
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, float scale, int causal, hipStream_t st);
hipError_t launch_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, float scale, int causal, hipStream_t st);
hipError_t launch_bwd_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                           int causal, void* ws, hipStream_t st);
hipError_t launch_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                              int N, int d, float scale, int causal, float p, unsigned long long seed,
                              bool fp16, hipStream_t st);
hipError_t launch_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                              int causal, float p, unsigned long long seed, void* ws, bool fp16, hipStream_t st);
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                          int N, int d, float scale, int causal, hipStream_t st);
hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                              int N, int d, float scale, int causal, int S, void* ws, bool fp16, hipStream_t st);
hipError_t launch_lse_merge(const float* op, const float* lp, int S, void* o, float* lse, int B, int H, int N,
                            int d, bool fp16, hipStream_t st);
hipError_t launch_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                             int d, float scale, int left, int right, bool fp16, hipStream_t st);
hipError_t launch_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                  int N, int d, float scale, int causal, const unsigned char* bm, int per_head,
                                  bool fp16, hipStream_t st);
hipError_t launch_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                             int left, int right, void* ws, bool fp16, hipStream_t st);
hipError_t launch_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                  float scale, int causal, const unsigned char* bm, int per_head, void* ws,
                                  bool fp16, hipStream_t st);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                      int causal, void* ws, hipStream_t st);
hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t st);
hipError_t launch_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                              int causal, hipStream_t st);

namespace {
// Per-device answer to "is this a gfx950?": 0 unknown, 1 yes, 2 no.  Written
// once per device; a benign cache of an immutable device property.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kErrDevice;
  if (dev < kMaxDevices) {
    const int known = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (known == 1) return kOk;
    if (known == 2) return kErrDevice;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return kErrDevice;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? kOk : kErrDevice;
}
}  // namespace
}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, float scale,
           int causal, hipStream_t stream) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_fwd(q, k, v, o, lse, s, scale, causal, 2);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, stream) == hipSuccess ? fa::kOk
                                                                                               : fa::kErrHip;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, hipStream_t stream) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_fwd(q, k, v, o, lse, s, scale, causal, 4);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream) == hipSuccess ? fa::kOk
                                                                                              : fa::kErrHip;
}

int fa_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                float scale, int causal, hipStream_t stream) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_fwd(q, k, v, o, lse, s, scale, causal, 2);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_fwd_fp16(q, k, v, o, lse, B, H, N, d, scale, causal, stream) == hipSuccess ? fa::kOk
                                                                                               : fa::kErrHip;
}

int fa_bwd_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_bwd(q, k, v, o, lse, dO, dq, dk, dv, s, scale, causal, workspace, workspace_bytes);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_bwd_fp16(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, workspace, stream) ==
                 hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

static int fa_fwd_dropout_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                               int d, float scale, int causal, float dropout_p, unsigned long long seed,
                               hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_fwd(q, k, v, o, lse, s, scale, causal, 2);
  if (st == fa::kOk) st = fa::check_dropout_p(dropout_p);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed, fp16, stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, float dropout_p, unsigned long long seed, hipStream_t stream) {
  return fa_fwd_dropout_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed, stream, false);
}

int fa_fwd_dropout_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                        float scale, int causal, float dropout_p, unsigned long long seed, hipStream_t stream) {
  return fa_fwd_dropout_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed, stream, true);
}

static int fa_bwd_dropout_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                               int causal, float dropout_p, unsigned long long seed, void* workspace,
                               size_t workspace_bytes, hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_bwd(q, k, v, o, lse, dO, dq, dk, dv, s, scale, causal, workspace, workspace_bytes);
  if (st == fa::kOk) st = fa::check_dropout_p(dropout_p);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_bwd_dropout(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, dropout_p, seed,
                                workspace, fp16, stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, float dropout_p,
                   unsigned long long seed, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_dropout_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, dropout_p, seed, workspace,
                             workspace_bytes, stream, false);
}

int fa_bwd_dropout_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                        void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                        float dropout_p, unsigned long long seed, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return fa_bwd_dropout_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, dropout_p, seed, workspace,
                             workspace_bytes, stream, true);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) { return fa::bwd_workspace_bytes(fa::Shape{B, H, N, d}); }

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_bwd(q, k, v, o, lse, dO, dq, dk, dv, s, scale, causal, workspace, workspace_bytes);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, workspace, stream) ==
                 hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                   hipStream_t stream) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, s, scale, causal);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
  return fa::split_workspace_bytes(fa::Shape{B, H, N, d}, num_splits);
}

int fa_fwd_splitkv_parts(int B, int H, int N, int d, int num_splits) {
  return fa::split_count(fa::Shape{B, H, N, d}, num_splits);
}

static int fa_fwd_splitkv_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                               int d, float scale, int causal, int num_splits, void* workspace,
                               size_t workspace_bytes, hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_fwd_splitkv(q, k, v, o, lse, s, scale, causal, num_splits, workspace, workspace_bytes);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  const int S = fa::split_count(s, num_splits);
  return fa::launch_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, S, workspace, fp16, stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, int num_splits, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  return fa_fwd_splitkv_impl(q, k, v, o, lse, B, H, N, d, scale, causal, num_splits, workspace, workspace_bytes,
                             stream, false);
}

int fa_fwd_splitkv_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                        float scale, int causal, int num_splits, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return fa_fwd_splitkv_impl(q, k, v, o, lse, B, H, N, d, scale, causal, num_splits, workspace, workspace_bytes,
                             stream, true);
}

static int fa_lse_merge_impl(const float* o_parts, const float* lse_parts, int num_parts, void* o, float* lse, int B,
                             int H, int N, int d, hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_lse_merge(o_parts, lse_parts, num_parts, o, lse, s);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_lse_merge(o_parts, lse_parts, num_parts, o, lse, B, H, N, d, fp16, stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_lse_merge(const float* o_parts, const float* lse_parts, int num_parts, void* o, float* lse, int B, int H,
                 int N, int d, hipStream_t stream) {
  return fa_lse_merge_impl(o_parts, lse_parts, num_parts, o, lse, B, H, N, d, stream, false);
}

int fa_lse_merge_fp16(const float* o_parts, const float* lse_parts, int num_parts, void* o, float* lse, int B, int H,
                      int N, int d, hipStream_t stream) {
  return fa_lse_merge_impl(o_parts, lse_parts, num_parts, o, lse, B, H, N, d, stream, true);
}

static int fa_fwd_window_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                              int d, float scale, int window_left, int window_right, hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_fwd_window(q, k, v, o, lse, s, scale);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_fwd_window(q, k, v, o, lse, B, H, N, d, scale, window_left, window_right, fp16, stream) ==
                 hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  float scale, int window_left, int window_right, hipStream_t stream) {
  return fa_fwd_window_impl(q, k, v, o, lse, B, H, N, d, scale, window_left, window_right, stream, false);
}

int fa_fwd_window_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                       float scale, int window_left, int window_right, hipStream_t stream) {
  return fa_fwd_window_impl(q, k, v, o, lse, B, H, N, d, scale, window_left, window_right, stream, true);
}

static int fa_fwd_blocksparse_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                   int N, int d, float scale, int causal, const unsigned char* block_mask,
                                   int mask_per_head, hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_fwd_blocksparse(q, k, v, o, lse, s, scale, causal, block_mask, mask_per_head);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, mask_per_head, fp16,
                                    stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                       float scale, int causal, const unsigned char* block_mask, int mask_per_head, hipStream_t stream
                       ) {
  return fa_fwd_blocksparse_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, mask_per_head, stream,
                                 false);
}

int fa_fwd_blocksparse_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                            int d, float scale, int causal, const unsigned char* block_mask, int mask_per_head,
                            hipStream_t stream) {
  return fa_fwd_blocksparse_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, mask_per_head, stream, true);
}

static int fa_bwd_window_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                              int window_left, int window_right, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, s, scale, workspace, workspace_bytes);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, window_left, window_right,
                               workspace, fp16, stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                  void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int window_left,
                  int window_right, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_window_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, window_left, window_right, workspace,
                            workspace_bytes, stream, false);
}

int fa_bwd_window_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int window_left,
                       int window_right, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_window_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, window_left, window_right, workspace,
                            workspace_bytes, stream, true);
}

static int fa_bwd_blocksparse_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                   float scale, int causal, const unsigned char* block_mask, int mask_per_head,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream, bool fp16) {
  const fa::Shape s{B, H, N, d};
  int st = fa::validate_bwd_blocksparse(q, k, v, o, lse, dO, dq, dk, dv, s, scale, causal, block_mask,
                                        mask_per_head, workspace, workspace_bytes);
  if (st != fa::kOk) return st;
  st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_bwd_blocksparse(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, block_mask,
                                    mask_per_head, workspace, fp16, stream) == hipSuccess
             ? fa::kOk
             : fa::kErrHip;
}

int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                       const unsigned char* block_mask, int mask_per_head, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return fa_bwd_blocksparse_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, block_mask,
                                 mask_per_head, workspace, workspace_bytes, stream, false);
}

int fa_bwd_blocksparse_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                            int causal, const unsigned char* block_mask, int mask_per_head, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_blocksparse_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, block_mask,
                                 mask_per_head, workspace, workspace_bytes, stream, true);
}

int fa_probe_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t stream) {
  if (!sink) return fa::kErrNull;
  if (workgroups < 1 || iters < 1 || workgroups > (1 << 20)) return fa::kErrArg;
  if (!fa::aligned16(sink)) return fa::kErrAlign;
  const int st = fa::check_device();
  if (st != fa::kOk) return st;
  return fa::launch_mfma_probe(workgroups, iters, sink, stream) == hipSuccess ? fa::kOk : fa::kErrHip;
}

const char* fa_status_string(int status) { return fa::status_string(status); }

}  // extern "C"
