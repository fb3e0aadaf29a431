"""The C ABI boundary, exercised on the host only (no GPU needed).

libfa2.so must load, export every function include/fa2.h declares, and reject
bad arguments before any HIP call: each check below returns before a kernel
could be enqueued, so no compute happens here.
"""
import ctypes
import math
import os
import re

import pytest

from exact_tiled_attention_30_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

OK, NULLPTR, SHAPE, HEADDIM, SCALE, ALIGN, ALIAS, WORKSPACE, LAUNCH, SCRATCH = range(10)

# Fake, well-aligned, non-overlapping "device" addresses.  Only argument
# checks run with them: every call below fails validation or is empty.
GB = 1 << 30
Q, K, V, O, LSE, DO, DQ, DK, DV, WS = (GB * (i + 1) for i in range(10))


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["fa2_bwd", "fa2_bwd_atomic_dq",
                                    "fa2_bwd_atomic_dq_workspace_bytes", "fa2_bwd_noalloc",
                                    "fa2_bwd_variant", "fa2_bwd_workspace_bytes",
                                    "fa2_calibrate_mfma", "fa2_calibrate_mfma_random",
                                    "fa2_fwd", "fa2_fwd_fa1_order",
                                    "fa2_fwd_fa1_order_workspace_bytes", "fa2_fwd_split_kv",
                                    "fa2_fwd_split_kv_workspace_bytes", "fa2_fwd_variant",
                                    "fa2_status_string", "fa2_variant_name"]


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), f"libfa2.so does not export {name}"


def test_status_strings(L):
    for s in range(10):
        msg = binding.fa2_status_string(s)
        assert msg.startswith("FA2_")
    assert binding.fa2_status_string(OK) == "FA2_OK"
    assert "unknown" in binding.fa2_status_string(99)


def fwd(L, q=Q, k=K, v=V, o=O, lse=LSE, B=2, H=3, N=100, d=64, causal=0, scale=0.125):
    return L.fa2_fwd(q, k, v, o, lse, B, H, N, d, causal, ctypes.c_float(scale), None)


def test_fwd_argument_errors(L):
    assert fwd(L, B=-1) == SHAPE
    assert fwd(L, H=-1) == SHAPE
    assert fwd(L, N=-5) == SHAPE
    assert fwd(L, d=96) == HEADDIM
    assert fwd(L, d=0) == HEADDIM
    assert fwd(L, scale=math.inf) == SCALE
    assert fwd(L, scale=math.nan) == SCALE
    # finite, but scale * log2(e) overflows fp32
    assert fwd(L, scale=3.0e38) == SCALE
    assert fwd(L, scale=-3.0e38) == SCALE
    # 2.3e38 * log2(e) is still finite: the shape checks pass and the NULL q fails
    assert fwd(L, q=None, scale=2.3e38) == NULLPTR
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd(L, **{name: None}) == NULLPTR, name
    for name in ("q", "k", "v", "o"):
        assert fwd(L, **{name: GB * 20 + 8}) == ALIGN, name
    assert fwd(L, lse=LSE + 2) == ALIGN
    # grid would exceed the launch limit
    assert fwd(L, B=1 << 20, H=1 << 10, N=1 << 20) == SHAPE
    # N above 2^30 (token indices plus a tile must stay inside int); at
    # exactly 2^30 the shape passes and the NULL q is what fails
    assert fwd(L, B=1, H=1, N=(1 << 30) + 1) == SHAPE
    assert fwd(L, B=1, H=1, N=2147483647) == SHAPE
    assert fwd(L, q=None, B=1, H=1, N=1 << 30) == NULLPTR
    # one token wider than 2^23 elements: in-tile row offsets would leave 32
    # bits.  At exactly 2^23 the shape passes and the NULL q is what fails.
    assert fwd(L, B=1, H=(1 << 16) + 1, N=8, d=128) == SHAPE
    assert fwd(L, B=1, H=(1 << 17) + 1, N=8, d=64) == SHAPE
    assert fwd(L, q=None, B=1, H=1 << 16, N=8, d=128) == NULLPTR
    assert fwd(L, q=None, B=1, H=1 << 17, N=8, d=64) == NULLPTR


def test_fwd_aliasing_is_rejected(L):
    assert fwd(L, o=Q) == ALIAS
    assert fwd(L, o=V + 64) == ALIAS         # o starts inside v
    assert fwd(L, lse=K + 128) == ALIAS       # lse inside k
    bytes_o = 2 * 3 * 100 * 64 * 2
    assert fwd(L, lse=O + bytes_o - 4) == ALIAS  # lse overlaps the tail of o


def test_fwd_empty_problem_is_a_noop(L):
    # B*H*N == 0 succeeds without touching any pointer (even NULL ones)
    assert fwd(L, q=None, k=None, v=None, o=None, lse=None, N=0) == OK
    assert fwd(L, q=None, k=None, v=None, o=None, lse=None, B=0) == OK
    assert fwd(L, q=None, k=None, v=None, o=None, lse=None, H=0) == OK
    # shape errors still win over the empty shortcut
    assert fwd(L, N=0, d=32) == HEADDIM


def test_bwd_workspace_size(L):
    for (B, H, N, d) in ((1, 1, 1, 64), (4, 16, 4096, 128), (2, 3, 257, 64)):
        want_d = (B * H * N * 4 + 255) // 256 * 256
        want_q = (B * H * N * d * 4 + 255) // 256 * 256
        assert binding.fa2_bwd_workspace_bytes(B, H, N, d, True) == want_d
        assert binding.fa2_bwd_atomic_dq_workspace_bytes(B, H, N, d, True) == want_d + want_q
    for f in (binding.fa2_bwd_workspace_bytes, binding.fa2_bwd_atomic_dq_workspace_bytes):
        assert f(0, 1, 1, 64, False) == 0
        assert f(1, 1, 1, 80, False) == 0
        assert f(-1, 1, 1, 64, False) == 0


def bwd(L, B=2, H=3, N=100, d=64, causal=1, scale=0.125, ws_bytes=None, atomic=False, **ptrs):
    p = dict(q=Q, k=K, v=V, o=O, lse=LSE, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS)
    p.update(ptrs)
    sizer = L.fa2_bwd_atomic_dq_workspace_bytes if atomic else L.fa2_bwd_workspace_bytes
    if ws_bytes is None:
        ws_bytes = sizer(B, H, N, d, causal)
    fn = L.fa2_bwd_atomic_dq if atomic else L.fa2_bwd
    return fn(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"], p["dv"],
              p["ws"], ws_bytes, B, H, N, d, causal, ctypes.c_float(scale), None)


@pytest.mark.parametrize("atomic", [False, True], ids=["two_pass", "atomic_dq"])
def test_bwd_argument_errors(L, atomic):
    assert bwd(L, N=-1, atomic=atomic) == SHAPE
    assert bwd(L, d=32, atomic=atomic) == HEADDIM
    assert bwd(L, scale=-math.inf, atomic=atomic) == SCALE
    for name in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"):
        assert bwd(L, atomic=atomic, **{name: None}) == NULLPTR, name
    assert bwd(L, ws=None, atomic=atomic) == WORKSPACE
    sizer = L.fa2_bwd_atomic_dq_workspace_bytes if atomic else L.fa2_bwd_workspace_bytes
    need = sizer(2, 3, 100, 64, 1)
    assert bwd(L, ws_bytes=need - 1, atomic=atomic) == WORKSPACE
    assert bwd(L, dq=DQ + 4, atomic=atomic) == ALIGN
    assert bwd(L, ws=WS + 8, atomic=atomic) == ALIGN
    assert bwd(L, dk=K, atomic=atomic) == ALIAS
    assert bwd(L, dv=DQ + 64, atomic=atomic) == ALIAS
    assert bwd(L, ws=DO, atomic=atomic) == ALIAS
    assert bwd(L, N=0, q=None, ws=None, atomic=atomic) == OK


def noalloc(L, B=2, H=3, N=100, d=64, causal=1, scale=0.125, **ptrs):
    p = dict(q=Q, k=K, v=V, o=O, lse=LSE, dout=DO, dq=DQ, dk=DK, dv=DV)
    p.update(ptrs)
    return L.fa2_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"],
                             p["dk"], p["dv"], B, H, N, d, causal, ctypes.c_float(scale), None)


def test_bwd_noalloc_argument_errors(L):
    # fa2_bwd's checks without a workspace, then the static scratch's limit;
    # every case returns before any HIP call
    assert noalloc(L, N=-1) == SHAPE
    assert noalloc(L, d=32) == HEADDIM
    assert noalloc(L, scale=math.nan) == SCALE
    for name in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"):
        assert noalloc(L, **{name: None}) == NULLPTR, name
    assert noalloc(L, dq=DQ + 4) == ALIGN
    assert noalloc(L, dk=K) == ALIAS
    assert noalloc(L, dv=DQ + 64) == ALIAS
    # one row past FA2_BWD_NOALLOC_MAX_ROWS (4 Mi rows of D, 16 MiB)
    assert binding.BWD_NOALLOC_MAX_ROWS == 4194304
    assert noalloc(L, B=1, H=1, N=4194305) == SCRATCH
    assert noalloc(L, B=2, H=4, N=524289, causal=0) == SCRATCH
    assert "FA2_BWD_NOALLOC_MAX_ROWS" in binding.fa2_status_string(SCRATCH)
    assert noalloc(L, N=0, q=None) == OK


def test_atomic_workspace_is_larger(L):
    # the two-pass backward's workspace is too small for the atomic one
    need = L.fa2_bwd_workspace_bytes(2, 3, 100, 64, 1)
    assert bwd(L, ws_bytes=need, atomic=True) == WORKSPACE


def fa1(L, q=Q, k=K, v=V, o=O, lse=LSE, ws=WS, ws_bytes=None, B=2, H=3, N=100, d=64, causal=0,
        scale=0.125):
    if ws_bytes is None:
        ws_bytes = L.fa2_fwd_fa1_order_workspace_bytes(B, H, N, d, causal)
    return L.fa2_fwd_fa1_order(q, k, v, o, lse, ws, ws_bytes, B, H, N, d, causal,
                               ctypes.c_float(scale), 0, None)


def test_fa1_order_argument_errors(L):
    B, H, N, d = 2, 3, 100, 64
    want = ((B * N * H * d * 4 + 255) // 256 * 256) + ((B * H * N * 8 + 255) // 256 * 256)
    assert L.fa2_fwd_fa1_order_workspace_bytes(B, H, N, d, 0) == want
    assert L.fa2_fwd_fa1_order_workspace_bytes(B, H, N, 80, 0) == 0
    assert fa1(L, d=96) == HEADDIM
    assert fa1(L, N=-1) == SHAPE
    assert fa1(L, scale=math.nan) == SCALE
    assert fa1(L, q=None) == NULLPTR
    assert fa1(L, ws=None) == WORKSPACE
    assert fa1(L, ws_bytes=want - 1) == WORKSPACE
    assert fa1(L, o=O + 2) == ALIGN
    assert fa1(L, ws=Q) == ALIAS
    assert fa1(L, o=K) == ALIAS
    assert fa1(L, N=0, q=None, ws=None) == OK


def split(L, q=Q, k=K, v=V, o=O, lse=LSE, ws=WS, ws_bytes=None, B=2, H=3, N=1000, d=64, causal=0,
          scale=0.125, n_split=0):
    if ws_bytes is None:
        ws_bytes = L.fa2_fwd_split_kv_workspace_bytes(B, H, N, d, causal, n_split)
    return L.fa2_fwd_split_kv(q, k, v, o, lse, ws, ws_bytes, B, H, N, d, causal,
                              ctypes.c_float(scale), n_split, None)


def test_split_kv_argument_errors(L):
    B, H, N, d = 2, 3, 1000, 64
    per = ((B * N * H * d * 4 + 255) // 256 * 256) + ((B * H * N * 4 + 255) // 256 * 256)
    assert L.fa2_fwd_split_kv_workspace_bytes(B, H, N, d, 0, 3) == 3 * per
    auto = L.fa2_fwd_split_kv_workspace_bytes(B, H, N, d, 0, 0)
    assert auto % per == 0 and 1 <= auto // per <= 16
    assert L.fa2_fwd_split_kv_workspace_bytes(B, H, N, d, 0, 65) == 0
    assert split(L, n_split=65) == SHAPE
    assert split(L, d=80) == HEADDIM
    assert split(L, ws=None) == WORKSPACE
    assert split(L, n_split=4, ws_bytes=4 * per - 1) == WORKSPACE
    assert split(L, lse=None) == NULLPTR
    assert split(L, ws=V) == ALIAS
    assert split(L, q=Q + 8) == ALIGN
    assert split(L, N=0, q=None, ws=None) == OK


def test_calibrate_mfma_argument_errors(L):
    # host-side validation only (no launch): a NULL buffer or a non-positive
    # size is rejected before any HIP call
    fake = ctypes.c_void_p(256)
    for fn in (L.fa2_calibrate_mfma, L.fa2_calibrate_mfma_random):
        assert fn(None, 1, 1, None) == 1          # FA2_ERR_NULLPTR
        assert fn(fake, 0, 1, None) == 2          # FA2_ERR_SHAPE
        assert fn(fake, 1, 0, None) == 2
