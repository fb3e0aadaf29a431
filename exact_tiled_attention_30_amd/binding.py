"""ctypes binding of libfa2.so -- argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into device pointers and sizes, picks the current torch
stream, and turns status codes into exceptions.  There is no fallback: if the
library is missing the call fails loudly.

Names mirror include/fa2.h: fa2_fwd, fa2_bwd, fa2_bwd_workspace_bytes, fa2_bwd_noalloc,
fa2_bwd_atomic_dq, fa2_bwd_atomic_dq_workspace_bytes, fa2_fwd_split_kv,
fa2_fwd_split_kv_workspace_bytes, fa2_fwd_fa1_order, fa2_fwd_fa1_order_workspace_bytes,
fa2_fwd_variant, fa2_bwd_variant, fa2_variant_name, fa2_calibrate_mfma,
fa2_calibrate_mfma_random, fa2_status_string.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa2.so")

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int


class Fa2Error(RuntimeError):
    """A nonzero fa2_status returned by the library."""

    def __init__(self, status: int):
        self.status = int(status)
        super().__init__(fa2_status_string(self.status))


def lib():
    """Load libfa2.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads the HIP runtime first

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m exact_tiled_attention_30_amd.build` "
            "(hipcc --offload-arch=gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    L.fa2_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float, _vp]
    L.fa2_fwd.restype = _i
    L.fa2_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    L.fa2_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.fa2_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                          _i, _i, _i, _i, _i, ctypes.c_float, _vp]
    L.fa2_bwd.restype = _i
    L.fa2_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                  _i, ctypes.c_float, _vp]
    L.fa2_bwd_noalloc.restype = _i
    L.fa2_bwd_atomic_dq_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    L.fa2_bwd_atomic_dq_workspace_bytes.restype = ctypes.c_size_t
    L.fa2_bwd_atomic_dq.argtypes = L.fa2_bwd.argtypes
    L.fa2_bwd_atomic_dq.restype = _i
    L.fa2_fwd_split_kv_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
    L.fa2_fwd_split_kv_workspace_bytes.restype = ctypes.c_size_t
    L.fa2_fwd_split_kv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i, _i, _i, _i,
                                   _i, ctypes.c_float, _i, _vp]
    L.fa2_fwd_split_kv.restype = _i
    L.fa2_fwd_fa1_order_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    L.fa2_fwd_fa1_order_workspace_bytes.restype = ctypes.c_size_t
    L.fa2_fwd_fa1_order.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i, _i, _i, _i,
                                    _i, ctypes.c_float, _i, _vp]
    L.fa2_fwd_fa1_order.restype = _i
    L.fa2_calibrate_mfma.argtypes = [_vp, _i, _i, _vp]
    L.fa2_calibrate_mfma.restype = _i
    L.fa2_calibrate_mfma_random.argtypes = [_vp, _i, _i, _vp]
    L.fa2_calibrate_mfma_random.restype = _i
    L.fa2_fwd_variant.argtypes = [_i, _i, _i, _i, _i, _i]
    L.fa2_fwd_variant.restype = _i
    L.fa2_bwd_variant.argtypes = [_i, _i, _i, _i, _i]
    L.fa2_bwd_variant.restype = _i
    L.fa2_variant_name.argtypes = [_i]
    L.fa2_variant_name.restype = ctypes.c_char_p
    L.fa2_status_string.argtypes = [_i]
    L.fa2_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def fa2_status_string(status: int) -> str:
    return lib().fa2_status_string(int(status)).decode()


def fa2_fwd_variant(B: int, H: int, N: int, d: int, causal: bool, resident_wgs: int = 0) -> int:
    """Id of the kernel configuration fa2_fwd launches (-1: invalid or empty);
    resident_wgs <= 0 asks the current device (see include/fa2.h)."""
    return int(lib().fa2_fwd_variant(B, H, N, d, int(bool(causal)), int(resident_wgs)))


def fa2_bwd_variant(B: int, H: int, N: int, d: int, causal: bool) -> int:
    """Id of the kernel configuration fa2_bwd launches (-1: invalid or empty)."""
    return int(lib().fa2_bwd_variant(B, H, N, d, int(bool(causal))))


def fa2_variant_name(variant: int) -> str:
    return lib().fa2_variant_name(int(variant)).decode()


def fa2_calibrate_mfma(out, blocks: int, iters: int, stream=None) -> None:
    """Measurement helper: `blocks` x 256 threads of back-to-back bf16 MFMAs
    (blocks x 4 x iters x 4 x 32768 FLOP); `out` a float32 device tensor of
    at least blocks x 256 elements.  Time it with events on `stream`."""
    _calibrate(lib().fa2_calibrate_mfma, out, blocks, iters, stream)


def fa2_calibrate_mfma_random(out, blocks: int, iters: int, stream=None) -> None:
    """As fa2_calibrate_mfma, with changing unit-variance random operands:
    the MFMA rate a power-capped GPU sustains on real data."""
    _calibrate(lib().fa2_calibrate_mfma_random, out, blocks, iters, stream)


def _calibrate(fn, out, blocks: int, iters: int, stream) -> None:
    import torch

    if out.dtype != torch.float32:
        raise TypeError(f"out must be {torch.float32}, got {out.dtype}")
    if out.numel() < blocks * 256:
        raise ValueError("out is too small")
    _require(out, torch.float32, "out")
    _check(fn(_ptr(out), int(blocks), int(iters), _stream(out, stream)))


def _check(status: int) -> None:
    if status != 0:
        raise Fa2Error(status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    import torch

    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _bnhd(q):
    if q.dim() != 4:
        raise ValueError("expected a [B, N, H, d] tensor")
    B, N, H, d = (int(x) for x in q.shape)
    return B, N, H, d


def _require(t, dtype, name):
    import torch

    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    del torch


def _shapes(named, lse, B, N, H, d):
    """Shapes first (they need no device): every [B, N, H, d] tensor, then lse
    [B, H, N] -- the kernels read B*H*N floats of it in that layout."""
    for t, name in named:
        if tuple(t.shape) != (B, N, H, d):
            raise ValueError(f"{name} must have shape {(B, N, H, d)}")
    if tuple(lse.shape) != (B, H, N):
        raise ValueError(f"lse must have shape {(B, H, N)}")


def _fwd_checks(q, k, v, o, lse):
    import torch

    B, N, H, d = _bnhd(q)
    named = ((q, "q"), (k, "k"), (v, "v"), (o, "o"))
    _shapes(named, lse, B, N, H, d)
    for t, name in named:
        _require(t, torch.bfloat16, name)
    _require(lse, torch.float32, "lse")
    return B, N, H, d


def fa2_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """Enqueue the forward pass on `stream` (default: torch's current stream).

    q, k, v, o: bf16 [B, N, H, d]; lse: fp32 [B, H, N].  Raises Fa2Error."""
    B, N, H, d = _fwd_checks(q, k, v, o, lse)
    _check(lib().fa2_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                         int(bool(causal)), float(scale), _stream(q, stream)))


def fa2_fwd_split_kv_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool,
                                     n_split: int = 0) -> int:
    return int(lib().fa2_fwd_split_kv_workspace_bytes(B, H, N, d, int(bool(causal)),
                                                       int(n_split)))


def fa2_fwd_split_kv(q, k, v, o, lse, workspace, causal: bool, scale: float, n_split: int = 0,
                     stream=None) -> None:
    """Enqueue the split-KV forward pass.  workspace: a uint8 device tensor of
    at least fa2_fwd_split_kv_workspace_bytes(..., n_split) bytes.  Raises Fa2Error."""
    import torch

    B, N, H, d = _fwd_checks(q, k, v, o, lse)
    _require(workspace, torch.uint8, "workspace")
    _check(lib().fa2_fwd_split_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                  workspace.numel(), B, H, N, d, int(bool(causal)), float(scale),
                                  int(n_split), _stream(q, stream)))


def fa2_fwd_fa1_order_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool) -> int:
    return int(lib().fa2_fwd_fa1_order_workspace_bytes(B, H, N, d, int(bool(causal))))


def fa2_fwd_fa1_order(q, k, v, o, lse, workspace, causal: bool, scale: float,
                      split_k: bool = False, stream=None) -> None:
    """Enqueue the forward pass in FlashAttention-1's loop order (an ablation);
    split_k: FlashAttention-1's own wave partition (waves split each K/V tile
    and merge through LDS) instead of FlashAttention-2's split-Q.  workspace:
    a uint8 device tensor of at least fa2_fwd_fa1_order_workspace_bytes(...)
    bytes.  Raises Fa2Error."""
    import torch

    B, N, H, d = _fwd_checks(q, k, v, o, lse)
    _require(workspace, torch.uint8, "workspace")
    _check(lib().fa2_fwd_fa1_order(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                   workspace.numel(), B, H, N, d, int(bool(causal)), float(scale),
                                   int(bool(split_k)), _stream(q, stream)))


def fa2_bwd_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool) -> int:
    return int(lib().fa2_bwd_workspace_bytes(B, H, N, d, int(bool(causal))))


def fa2_bwd_atomic_dq_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool) -> int:
    return int(lib().fa2_bwd_atomic_dq_workspace_bytes(B, H, N, d, int(bool(causal))))


def _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, scale, stream):
    import torch

    B, N, H, d = _bnhd(q)
    named = ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
             (dv, "dv"))
    _shapes(named, lse, B, N, H, d)
    for t, name in named:
        _require(t, torch.bfloat16, name)
    _require(lse, torch.float32, "lse")
    _require(workspace, torch.uint8, "workspace")
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace.numel(), B, H, N, d, int(bool(causal)),
            float(scale), _stream(q, stream))


def fa2_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal: bool, scale: float,
            stream=None) -> None:
    """Enqueue the backward pass (dQ from a Q-outer pass). workspace: a uint8
    device tensor of at least fa2_bwd_workspace_bytes(...) bytes.  Raises Fa2Error."""
    _check(lib().fa2_bwd(*_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, scale,
                                     stream)))


BWD_NOALLOC_MAX_ROWS = 4194304  # FA2_BWD_NOALLOC_MAX_ROWS of include/fa2.h


def fa2_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, scale: float,
                    stream=None) -> None:
    """Enqueue fa2_bwd with the library's static scratch instead of a
    workspace: no device memory is allocated (B*H*N <= BWD_NOALLOC_MAX_ROWS;
    calls overlapping on one GPU race).  Raises Fa2Error."""
    import torch

    B, N, H, d = _bnhd(q)
    named = ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
             (dv, "dv"))
    _shapes(named, lse, B, N, H, d)
    for t, name in named:
        _require(t, torch.bfloat16, name)
    _require(lse, torch.float32, "lse")
    _check(lib().fa2_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)),
                                 float(scale), _stream(q, stream)))


def fa2_bwd_atomic_dq(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal: bool, scale: float,
                      stream=None) -> None:
    """Enqueue the backward pass with dQ summed by fp32 atomics. workspace: at
    least fa2_bwd_atomic_dq_workspace_bytes(...) bytes.  Raises Fa2Error."""
    _check(lib().fa2_bwd_atomic_dq(*_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal,
                                               scale, stream)))


# ---- conveniences that allocate the outputs with torch, then call the above

def attention_forward(q, k, v, causal: bool = False, scale: float | None = None):
    """Allocate O and L, run fa2_fwd, return (o, lse)."""
    import torch

    B, N, H, d = _bnhd(q)
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa2_fwd(q, k, v, o, lse, causal, scale)
    return o, lse


def attention_forward_split_kv(q, k, v, causal: bool = False, scale: float | None = None,
                               n_split: int = 0):
    """Allocate O, L and the workspace, run fa2_fwd_split_kv, return (o, lse)."""
    import torch

    B, N, H, d = _bnhd(q)
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, fa2_fwd_split_kv_workspace_bytes(B, H, N, d, causal, n_split)),
                     dtype=torch.uint8, device=q.device)
    fa2_fwd_split_kv(q, k, v, o, lse, ws, causal, scale, n_split)
    return o, lse


def attention_forward_fa1_order(q, k, v, causal: bool = False, scale: float | None = None,
                                split_k: bool = False):
    """Allocate O, L and the workspace, run fa2_fwd_fa1_order, return (o, lse)."""
    import torch

    B, N, H, d = _bnhd(q)
    if scale is None:
        scale = d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, fa2_fwd_fa1_order_workspace_bytes(B, H, N, d, causal)),
                     dtype=torch.uint8, device=q.device)
    fa2_fwd_fa1_order(q, k, v, o, lse, ws, causal, scale, split_k)
    return o, lse


def attention_backward(q, k, v, o, lse, dout, causal: bool = False,
                       scale: float | None = None, atomic_dq: bool = False):
    """Allocate dQ, dK, dV and the workspace, run fa2_bwd (or fa2_bwd_atomic_dq),
    return (dq, dk, dv)."""
    import torch

    B, N, H, d = _bnhd(q)
    if scale is None:
        scale = d ** -0.5
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    sizer = fa2_bwd_atomic_dq_workspace_bytes if atomic_dq else fa2_bwd_workspace_bytes
    ws = torch.empty(max(1, sizer(B, H, N, d, causal)), dtype=torch.uint8, device=q.device)
    (fa2_bwd_atomic_dq if atomic_dq else fa2_bwd)(q, k, v, o, lse, dout, dq, dk, dv, ws, causal,
                                                 scale)
    return dq, dk, dv
