"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/fa.h declares, and rejects invalid arguments before touching the GPU.

No call here reaches a kernel: every call fails validation, which runs before
the device check and before anything is enqueued.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "aware_exact_attention_amd", "libfa.so")

ST = {"OK": 0, "NULL": -1, "SHAPE": -2, "HEAD_DIM": -3, "SCALE": -4, "ALIGN": -5, "WORKSPACE": -6,
      "DEVICE": -7, "HIP": -8, "ARG": -9, "SCRATCH": -10}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import aware_exact_attention_amd.build as b
        b.build()
    from aware_exact_attention_amd import fa
    return fa.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["fa_fwd", "fa_fwd_f32", "fa_bwd_workspace_bytes", "fa_bwd", "fa_bwd_noalloc", "fa_probe_mfma_bf16",
                                           "fa_fwd_fp16", "fa_bwd_fp16", "fa_fwd_dropout", "fa_bwd_dropout",
                                           "fa_fwd_splitkv_parts", "fa_fwd_splitkv_workspace_bytes",
                                           "fa_fwd_splitkv", "fa_lse_merge", "fa_fwd_window",
                                           "fa_fwd_blocksparse", "fa_bwd_window", "fa_bwd_blocksparse",
                                           "fa_fwd_splitkv_fp16", "fa_lse_merge_fp16", "fa_fwd_window_fp16",
                                           "fa_bwd_window_fp16", "fa_fwd_blocksparse_fp16", "fa_bwd_blocksparse_fp16",
                                           "fa_fwd_dropout_fp16", "fa_bwd_dropout_fp16", "fa_status_string"])


def test_library_exports_every_declared_symbol(lib):
    from aware_exact_attention_amd import fa
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, f"{name} not exported by libfa.so"
        assert name in fa.SIGNATURES
        assert hasattr(lib, name)


def test_status_codes_match_header(lib):
    text = open(HEADER).read()
    for name, val in ST.items():
        assert re.search(rf"FA_(ERR_)?{name}\s*=\s*{val}\b", text), name
    for val in ST.values():
        s = lib.fa_status_string(val).decode()
        assert s and s != "unknown fa_status"
    assert lib.fa_status_string(12345).decode() == "unknown fa_status"


class _Buf:
    """Host buffers used only as distinct, aligned, non-null addresses."""

    def __init__(self, nbytes):
        self.raw = ctypes.create_string_buffer(nbytes + 64)
        a = ctypes.addressof(self.raw)
        self.ptr = (a + 15) // 16 * 16


def _fwd_args(B=1, H=1, N=8, d=64):
    bufs = [_Buf(B * H * N * d * 4) for _ in range(4)] + [_Buf(B * H * N * 4)]
    return bufs, [b.ptr for b in bufs]


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32", "fa_fwd_fp16"])
def test_fwd_validation(lib, fn):
    f = getattr(lib, fn)
    bufs, (q, k, v, o, l) = _fwd_args()
    assert f(None, k, v, o, l, 1, 1, 8, 64, 0.125, 0, None) == ST["NULL"]
    assert f(q, k, v, o, None, 1, 1, 8, 64, 0.125, 0, None) == ST["NULL"]
    assert f(q, k, v, o, l, 0, 1, 8, 64, 0.125, 0, None) == ST["SHAPE"]
    assert f(q, k, v, o, l, 1, -1, 8, 64, 0.125, 0, None) == ST["SHAPE"]
    assert f(q, k, v, o, l, 1, 1, 0, 64, 0.125, 0, None) == ST["SHAPE"]
    assert f(q, k, v, o, l, 1 << 12, 1 << 10, 1 << 10, 64, 0.125, 0, None) == ST["SHAPE"]
    assert f(q, k, v, o, l, 1, 1, (1 << 22) - 256, 128, 0.125, 0, None) == ST["SHAPE"]  # one head > 2^31 B fp32
    assert f(q, k, v, o, l, 1, 1, 8, 80, 0.125, 0, None) == ST["HEAD_DIM"]
    assert f(q, k, v, o, l, 1, 1, 8, 512, 0.125, 0, None) == ST["HEAD_DIM"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, float("nan"), 0, None) == ST["SCALE"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, float("inf"), 0, None) == ST["SCALE"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, 0.0, 0, None) == ST["SCALE"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, -0.125, 0, None) == ST["SCALE"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, 0.125, 2, None) == ST["ARG"]
    assert f(q + 2, k, v, o, l, 1, 1, 8, 64, 0.125, 0, None) == ST["ALIGN"]
    assert f(q, k, v, o, l + 4, 1, 1, 8, 64, 0.125, 0, None) == ST["ALIGN"]
    assert f(q, k, v, q, l, 1, 1, 8, 64, 0.125, 0, None) == ST["ARG"]  # output aliases input
    assert f(q, k, v, o, o, 1, 1, 8, 64, 0.125, 0, None) == ST["ARG"]  # lse aliases output


def test_bwd_workspace_bytes(lib):
    n = 2 * 3 * 100 * 128
    want = 2 * ((2 * 3 * 100 * 4 + 255) // 256 * 256)
    assert lib.fa_bwd_workspace_bytes(2, 3, 100, 128) == want
    assert lib.fa_bwd_workspace_bytes(0, 3, 100, 128) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 100, 80) == 0


@pytest.mark.parametrize("fn", ["fa_bwd", "fa_bwd_fp16"])
def test_bwd_validation(lib, fn):
    B, H, N, d = 1, 2, 16, 64
    bufs = [_Buf(B * H * N * d * 2) for _ in range(9)]
    q, k, v, o, lse, do, dq, dk, dv = [b.ptr for b in bufs]
    need = lib.fa_bwd_workspace_bytes(B, H, N, d)
    wsb = _Buf(need)
    ws = wsb.ptr
    base = [q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, 0.125, 1, ws, need, None]

    def call(**ch):
        a = list(base)
        names = ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "B", "H", "N", "d", "scale", "causal", "ws",
                 "wsb", "stream"]
        for kk, vv in ch.items():
            a[names.index(kk)] = vv
        return getattr(lib, fn)(*a)

    assert call(do=None) == ST["NULL"]
    assert call(dk=None) == ST["NULL"]
    assert call(N=0) == ST["SHAPE"]
    assert call(d=32) == ST["HEAD_DIM"]
    assert call(d=512) == ST["HEAD_DIM"]  # d = 256 is accepted (every entry point)
    assert call(scale=float("nan")) == ST["SCALE"]
    assert call(causal=-1) == ST["ARG"]
    assert call(ws=None) == ST["WORKSPACE"]
    assert call(wsb=need - 1) == ST["WORKSPACE"]
    assert call(dq=dq + 8) == ST["ALIGN"]
    assert call(dk=dq) == ST["ARG"]          # two outputs alias
    assert call(dv=v) == ST["ARG"]           # output aliases an input
    assert call(ws=dq) == ST["ARG"]          # workspace aliases an output


def test_bwd_noalloc_validation(lib):
    """fa_bwd_noalloc takes fa_bwd's arguments minus the workspace; a problem
    whose workspace exceeds the library's 32 MiB scratch is refused before
    anything is enqueued (4194304 rows fit, one more does not)."""
    B, H, N, d = 1, 2, 16, 64
    bufs = [_Buf(B * H * N * d * 2) for _ in range(9)]
    q, k, v, o, lse, do, dq, dk, dv = [b.ptr for b in bufs]
    f = lib.fa_bwd_noalloc
    assert f(q, k, v, o, lse, None, dq, dk, dv, B, H, N, d, 0.125, 1, None) == ST["NULL"]
    assert f(q, k, v, o, lse, do, dq, dk, dv, B, H, 0, d, 0.125, 1, None) == ST["SHAPE"]
    assert f(q, k, v, o, lse, do, dq, dk, dv, B, H, N, 80, 0.125, 1, None) == ST["HEAD_DIM"]
    assert f(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, -1.0, 1, None) == ST["SCALE"]
    assert f(q, k, v, o, lse, do, dq + 4, dk, dv, B, H, N, d, 0.125, 1, None) == ST["ALIGN"]
    assert f(q, k, v, o, lse, do, dq, dq, dv, B, H, N, d, 0.125, 1, None) == ST["ARG"]
    assert f(q, k, v, o, lse, do, dq, dk, k, B, H, N, d, 0.125, 1, None) == ST["ARG"]
    assert f(q, k, v, o, lse, do, dq, dk, dv, 1, 64, 65537, 64, 0.125, 0, None) == ST["SCRATCH"]
    assert f(q, k, v, o, lse, do, dq, dk, dv, 1, 1, (1 << 22) + 1, 64, 0.125, 0, None) == ST["SCRATCH"]
    assert lib.fa_bwd_workspace_bytes(1, 64, 65536, 64) == 32 << 20
    assert lib.fa_bwd_workspace_bytes(1, 64, 65537, 64) > 32 << 20


def test_probe_validation(lib):
    b = _Buf(4096)
    assert lib.fa_probe_mfma_bf16(1, 1, None, None) == ST["NULL"]
    assert lib.fa_probe_mfma_bf16(0, 1, b.ptr, None) == ST["ARG"]
    assert lib.fa_probe_mfma_bf16(1, 0, b.ptr, None) == ST["ARG"]
    assert lib.fa_probe_mfma_bf16(1, 1, b.ptr + 4, None) == ST["ALIGN"]


def test_splitkv_parts_and_workspace(lib):
    parts = lib.fa_fwd_splitkv_parts
    # automatic: 8 heads of 16 query blocks = 128 workgroups -> 4 parts reach 512
    assert parts(1, 8, 2048, 128, 0) == 4
    assert parts(1, 8, 16384, 128, 0) == 1      # 1024 workgroups already
    assert parts(1, 1, 256, 64, 0) == 2         # 4 tiles: at least two per part
    assert parts(1, 1, 64, 64, 0) == 1          # one tile
    assert parts(1, 1, 4096, 64, 0) == 16       # 32 workgroups, 64 tiles: 16 parts of 4
    assert parts(1, 1, 2816, 64, 0) == 15       # wants 24, capped at 16: 44 tiles in parts of 3 fill 15
    assert parts(1, 1, 8192, 64, 0) == 8        # 64 workgroups
    # requests: capped at the tile count, parts without tiles dropped
    assert parts(1, 8, 2048, 128, 5) == 5       # 32 tiles: 7,7,7,7,4
    assert parts(1, 1, 640, 64, 100) == 10
    assert parts(1, 1, 576, 64, 4) == 3         # 9 tiles, 3 per part
    assert parts(1, 1, 1 << 20, 64, 1000) == 64
    assert parts(0, 1, 64, 64, 2) == 0 and parts(1, 1, 64, 80, 2) == 0
    ws = lib.fa_fwd_splitkv_workspace_bytes
    rows = 8 * 2048
    assert ws(1, 8, 2048, 128, 0) == 4 * rows * 128 * 4 + 4 * rows * 4
    assert ws(1, 8, 16384, 128, 0) == 0
    assert ws(1, 1, 100, 64, 2) == (2 * 100 * 64 * 4 + 255) // 256 * 256 + (2 * 100 * 4 + 255) // 256 * 256
    assert ws(1, 1, 100, 80, 2) == 0


def test_splitkv_validation(lib):
    B, H, N, d = 1, 1, 256, 64
    bufs = [_Buf(B * H * N * d * 2) for _ in range(4)] + [_Buf(B * H * N * 4)]
    q, k, v, o, l = [b.ptr for b in bufs]
    need = lib.fa_fwd_splitkv_workspace_bytes(B, H, N, d, 2)
    assert need > 0
    wsb = _Buf(need)
    f = lib.fa_fwd_splitkv
    assert f(None, k, v, o, l, B, H, N, d, 0.125, 0, 2, wsb.ptr, need, None) == ST["NULL"]
    assert f(q, k, v, o, l, B, H, N, 80, 0.125, 0, 2, wsb.ptr, need, None) == ST["HEAD_DIM"]
    assert f(q, k, v, o, l, B, H, N, d, 0.0, 0, 2, wsb.ptr, need, None) == ST["SCALE"]
    assert f(q, k, v, o, l, B, H, N, d, 0.125, 3, 2, wsb.ptr, need, None) == ST["ARG"]
    assert f(q, k, v, o, l, B, H, N, d, 0.125, 0, 2, None, 0, None) == ST["WORKSPACE"]
    assert f(q, k, v, o, l, B, H, N, d, 0.125, 0, 2, wsb.ptr, need - 1, None) == ST["WORKSPACE"]
    assert f(q, k, v, o, l, B, H, N, d, 0.125, 0, 2, wsb.ptr + 8, need, None) == ST["ALIGN"]
    assert f(q, k, v, o, l, B, H, N, d, 0.125, 0, 2, o, need, None) == ST["ARG"]  # workspace over an output


def test_lse_merge_validation(lib):
    S, B, H, N, d = 3, 1, 2, 8, 64
    op, lp = _Buf(S * B * H * N * d * 4), _Buf(S * B * H * N * 4)
    o, l = _Buf(B * H * N * d * 2), _Buf(B * H * N * 4)
    f = lib.fa_lse_merge
    assert f(None, lp.ptr, S, o.ptr, l.ptr, B, H, N, d, None) == ST["NULL"]
    assert f(op.ptr, lp.ptr, S, o.ptr, None, B, H, N, d, None) == ST["NULL"]
    assert f(op.ptr, lp.ptr, S, o.ptr, l.ptr, B, 0, N, d, None) == ST["SHAPE"]
    assert f(op.ptr, lp.ptr, S, o.ptr, l.ptr, B, H, N, 32, None) == ST["HEAD_DIM"]
    assert f(op.ptr, lp.ptr, 0, o.ptr, l.ptr, B, H, N, d, None) == ST["ARG"]
    assert f(op.ptr, lp.ptr, 5000, o.ptr, l.ptr, B, H, N, d, None) == ST["ARG"]
    assert f(op.ptr + 4, lp.ptr, S, o.ptr, l.ptr, B, H, N, d, None) == ST["ALIGN"]
    assert f(op.ptr, lp.ptr, S, op.ptr + 64, l.ptr, B, H, N, d, None) == ST["ARG"]  # output inside the parts
    assert f(op.ptr, lp.ptr, S, o.ptr, o.ptr, B, H, N, d, None) == ST["ARG"]        # lse over o


def test_mask_validation(lib):
    B, H, N, d = 1, 2, 130, 64
    bufs = [_Buf(B * H * N * d * 2) for _ in range(4)] + [_Buf(B * H * N * 4)]
    q, k, v, o, l = [b.ptr for b in bufs]
    fw = lib.fa_fwd_window
    assert fw(None, k, v, o, l, B, H, N, d, 0.125, 4, 4, None) == ST["NULL"]
    assert fw(q, k, v, o, l, B, H, N, 80, 0.125, 4, 4, None) == ST["HEAD_DIM"]
    assert fw(q, k, v, o, l, B, H, N, d, -1.0, 4, 4, None) == ST["SCALE"]
    assert fw(q, k, v, q, l, B, H, N, d, 0.125, 4, 4, None) == ST["ARG"]
    nb = 3
    m = _Buf(H * nb * nb)
    fb = lib.fa_fwd_blocksparse
    assert fb(q, k, v, o, l, B, H, N, d, 0.125, 0, None, 1, None) == ST["NULL"]
    assert fb(q, k, v, o, l, B, H, 65537, d, 0.125, 0, m.ptr, 1, None) == ST["SHAPE"]
    assert fb(q, k, v, o, l, B, H, N, d, 0.125, 2, m.ptr, 1, None) == ST["ARG"]
    assert fb(q, k, v, o, l, B, H, N, d, 0.125, 0, m.ptr, 2, None) == ST["ARG"]
    assert fb(q, k, v, o, l, B, H, N, d, 0.125, 0, o, 1, None) == ST["ARG"]      # mask overlaps the output
    # masked backward: fa_bwd's checks plus the mask's
    bb = [_Buf(B * H * N * d * 2) for _ in range(9)]
    ptrs = [b.ptr for b in bb]
    need = lib.fa_bwd_workspace_bytes(B, H, N, d)
    ws = _Buf(need)
    gw = lib.fa_bwd_window
    assert gw(None, *ptrs[1:], B, H, N, d, 0.125, 4, 4, ws.ptr, need, None) == ST["NULL"]
    assert gw(*ptrs, B, H, N, 80, 0.125, 4, 4, ws.ptr, need, None) == ST["HEAD_DIM"]
    assert gw(*ptrs, B, H, N, d, 0.125, 4, 4, None, 0, None) == ST["WORKSPACE"]
    assert gw(*ptrs, B, H, N, d, 0.125, 4, 4, ws.ptr, need - 1, None) == ST["WORKSPACE"]
    assert gw(*ptrs[:6], ptrs[0], *ptrs[7:], B, H, N, d, 0.125, 4, 4, ws.ptr, need, None) == ST["ARG"]  # dq over q
    gb = lib.fa_bwd_blocksparse
    assert gb(*ptrs, B, H, N, d, 0.125, 0, None, 1, ws.ptr, need, None) == ST["NULL"]
    assert gb(*ptrs, B, H, 65537, d, 0.125, 0, m.ptr, 1, ws.ptr, need, None) in (ST["SHAPE"], ST["WORKSPACE"])
    assert gb(*ptrs, B, H, N, d, 0.125, 2, m.ptr, 1, ws.ptr, need, None) == ST["ARG"]
    assert gb(*ptrs, B, H, N, d, 0.125, 0, m.ptr, 2, ws.ptr, need, None) == ST["ARG"]
    assert gb(*ptrs, B, H, N, d, 0.125, 0, ptrs[7], 1, ws.ptr, need, None) == ST["ARG"]  # mask overlaps dk
    assert gb(*ptrs, B, H, N, d, 0.125, 0, m.ptr, 1, None, 0, None) == ST["WORKSPACE"]


def test_dropout_validation(lib):
    bufs, (q, k, v, o, l) = _fwd_args()
    f = lib.fa_fwd_dropout
    assert f(None, k, v, o, l, 1, 1, 8, 64, 0.125, 0, 0.1, 7, None) == ST["NULL"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, 0.125, 0, -0.1, 7, None) == ST["ARG"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, 0.125, 0, 1.0, 7, None) == ST["ARG"]
    assert f(q, k, v, o, l, 1, 1, 8, 64, 0.125, 0, float("nan"), 7, None) == ST["ARG"]
    assert f(q, k, v, o, l, 1, 1, 8, 80, 0.125, 0, 0.1, 7, None) == ST["HEAD_DIM"]
    B, H, N, d = 1, 2, 16, 64
    bb = [_Buf(B * H * N * d * 2) for _ in range(9)]
    ptrs = [b.ptr for b in bb]
    need = lib.fa_bwd_workspace_bytes(B, H, N, d)
    ws = _Buf(need)
    g = lib.fa_bwd_dropout
    assert g(*ptrs, B, H, N, d, 0.125, 0, 1.5, 7, ws.ptr, need, None) == ST["ARG"]
    assert g(*ptrs, B, H, N, d, 0.125, 0, 0.2, 7, None, 0, None) == ST["WORKSPACE"]


def test_validate_header_with_gxx(tmp_path):
    """Host unit test of fa_validate.h compiled by g++ (no HIP, no GPU)."""
    src = tmp_path / "t.cpp"
    src.write_text(r'''
#include "fa_validate.h"
#include <cstdio>
#include <cmath>
using namespace fa;
static int fails = 0;
#define EXPECT(x) do { if (!(x)) { std::printf("FAIL line %d: %s\n", __LINE__, #x); ++fails; } } while (0)
int main() {
  alignas(16) static char mem[10][8192];
  alignas(16) static char ws[1 << 16];
  Shape s{1, 2, 16, 64};
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[3], mem[4], s, 0.125f, 0, 2) == kOk);
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[3], mem[4], s, 0.125f, 1, 4) == kOk);
  EXPECT(validate_fwd(nullptr, mem[1], mem[2], mem[3], mem[4], s, 0.125f, 0, 2) == kErrNull);
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[3], mem[4], Shape{1, 2, 16, 65}, 0.125f, 0, 2) == kErrHeadDim);
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[3], mem[4], Shape{1, 0, 16, 64}, 0.125f, 0, 2) == kErrShape);
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[3], mem[4], s, NAN, 0, 2) == kErrScale);
  EXPECT(validate_fwd(mem[0] + 1, mem[1], mem[2], mem[3], mem[4], s, 0.125f, 0, 2) == kErrAlign);
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[0] + 16, mem[4], s, 0.125f, 0, 2) == kErrArg);
  EXPECT(tensor_elems(Shape{1024, 1024, 1024, 2}) == -1);
  EXPECT(tensor_elems(Shape{2, 3, 5, 64}) == 1920);
  size_t need = bwd_workspace_bytes(s);
  EXPECT(need == 256 + 256);
  EXPECT(bwd_workspace_layout(s).d == 0 && bwd_workspace_layout(s).lse2 == 256);
  EXPECT(tensor_elems(Shape{1, 1, (1 << 22) - 256, 128}) == -1);
  EXPECT(tensor_elems(Shape{1, 1, (1 << 22) - 257, 128}) > 0);
  EXPECT(validate_bwd(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s, 0.125f, 1,
                      ws, sizeof ws) == kOk);
  EXPECT(validate_bwd(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s, 0.125f, 1,
                      ws, need - 1) == kErrWorkspace);
  EXPECT(validate_bwd(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[6], mem[8], s, 0.125f, 1,
                      ws, sizeof ws) == kErrArg);
  EXPECT(overlaps(mem[0], 16, mem[0] + 15, 1) && !overlaps(mem[0], 16, mem[0] + 16, 1));
  EXPECT(split_count(Shape{1, 8, 2048, 128}, 0) == 4);
  EXPECT(split_count(Shape{1, 8, 2048, 128}, 1) == 1);
  EXPECT(split_count(Shape{1, 1, 576, 64}, 4) == 3);
  EXPECT(split_count(Shape{1, 1, 64, 65}, 2) == 0);
  EXPECT(split_workspace_layout(s, 1).total == 0);
  EXPECT(split_workspace_layout(s, 2).lse_parts == 2 * 32 * 64 * 4);
  EXPECT(split_workspace_layout(s, 2).total == 2 * 32 * 64 * 4 + 256);
  EXPECT(validate_fwd_splitkv(mem[0], mem[1], mem[2], mem[3], mem[4], s, 0.125f, 0, 1, nullptr, 0) == kOk);
  alignas(16) static char big[6][65536];
  const Shape s2{1, 1, 256, 64};
  const size_t need2 = split_workspace_layout(s2, 2).total;
  EXPECT(need2 == 2 * 256 * 64 * 4 + 2 * 256 * 4);
  EXPECT(validate_fwd_splitkv(big[0], big[1], big[2], big[3], big[4], s2, 0.125f, 0, 2, nullptr, 0) == kErrWorkspace);
  EXPECT(validate_fwd_splitkv(big[0], big[1], big[2], big[3], big[4], s2, 0.125f, 0, 2, big[5], 65536) == kErrWorkspace);
  EXPECT(need2 > 65536);  // so the 64 KiB buffer above is too small
  EXPECT(validate_lse_merge(mem[0], mem[1], 2, mem[2], mem[3], Shape{1, 1, 8, 64}) == kOk);
  EXPECT(validate_lse_merge(mem[0], mem[1], 0, mem[2], mem[3], Shape{1, 1, 8, 64}) == kErrArg);
  EXPECT(validate_lse_merge(mem[0], mem[1], 2, mem[0] + 64, mem[3], Shape{1, 1, 8, 64}) == kErrArg);
  EXPECT(block_mask_bytes(Shape{1, 3, 130, 64}, 1) == 27 && block_mask_bytes(Shape{1, 3, 130, 64}, 0) == 9);
  EXPECT(validate_fwd_blocksparse(mem[0], mem[1], mem[2], mem[3], mem[4], s, 0.125f, 1, mem[5], 1) == kOk);
  EXPECT(validate_fwd_blocksparse(mem[0], mem[1], mem[2], mem[3], mem[4], s, 0.125f, 1, nullptr, 1) == kErrNull);
  EXPECT(validate_fwd_blocksparse(mem[0], mem[1], mem[2], mem[3], mem[4], s, 0.125f, 1, mem[3], 1) == kErrArg);
  EXPECT(validate_fwd_window(mem[0], mem[1], mem[2], mem[3], mem[4], s, 0.125f) == kOk);
  EXPECT(validate_bwd_window(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s, 0.125f,
                             ws, sizeof ws) == kOk);
  EXPECT(validate_bwd_blocksparse(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s,
                                  0.125f, 1, mem[9], 1, ws, sizeof ws) == kOk);
  EXPECT(validate_bwd_blocksparse(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s,
                                  0.125f, 1, nullptr, 1, ws, sizeof ws) == kErrNull);
  EXPECT(validate_bwd_blocksparse(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s,
                                  0.125f, 1, mem[6], 1, ws, sizeof ws) == kErrArg);
  EXPECT(validate_bwd_blocksparse(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s,
                                  0.125f, 1, mem[9], 3, ws, sizeof ws) == kErrArg);
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[3], mem[4], Shape{1, 1, 8, 256}, 0.125f, 0, 2) == kOk);
  EXPECT(validate_fwd(mem[0], mem[1], mem[2], mem[3], mem[4], Shape{1, 1, 8, 96}, 0.125f, 0, 2) == kOk);
  // d = 256 on every backward entry point; 512 nowhere
  EXPECT(validate_bwd(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], Shape{1, 1, 8, 256},
                      0.125f, 1, ws, sizeof ws) == kOk);
  EXPECT(validate_bwd(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], Shape{1, 1, 8, 512},
                      0.125f, 1, ws, sizeof ws) == kErrHeadDim);
  EXPECT(validate_bwd_window(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8],
                             Shape{1, 1, 8, 256}, 0.125f, ws, sizeof ws) == kOk);
  EXPECT(bwd_workspace_bytes(Shape{1, 1, 8, 256}) == 512 && bwd_workspace_bytes(Shape{1, 1, 8, 96}) == 512);
  EXPECT(bwd_workspace_bytes(Shape{1, 1, 8, 512}) == 0);
  EXPECT(split_count(Shape{1, 1, 256, 256}, 2) == 2);
  EXPECT(validate_lse_merge(mem[0], mem[1], 2, mem[2], mem[3], Shape{1, 1, 8, 256}) == kOk);
  EXPECT(validate_bwd_noalloc(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8], s, 0.125f,
                              1) == kOk);
  EXPECT(validate_bwd_noalloc(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[6], mem[8], s, 0.125f,
                              1) == kErrArg);
  EXPECT(validate_bwd_noalloc(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8],
                              Shape{1, 64, 65536, 64}, 0.125f, 1) != kErrScratch);
  EXPECT(validate_bwd_noalloc(mem[0], mem[1], mem[2], mem[3], mem[4], mem[5], mem[6], mem[7], mem[8],
                              Shape{1, 64, 65537, 64}, 0.125f, 1) == kErrScratch);
  EXPECT(check_dropout_p(0.0f) == kOk && check_dropout_p(0.999f) == kOk);
  EXPECT(check_dropout_p(1.0f) == kErrArg && check_dropout_p(-1e-9f) == kErrArg && check_dropout_p(NAN) == kErrArg);
  return fails ? 1 : 0;
}
''')
    exe = tmp_path / "t"
    inc = os.path.join(ROOT, "aware_exact_attention_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-fsanitize=address,undefined", "-I", inc, str(src),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
