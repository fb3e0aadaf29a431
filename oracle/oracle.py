"""ctypes front end of oracle.c, the plain fp64 attention reference.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  Inputs (numpy arrays or CPU torch
tensors of any float dtype, including bfloat16) are widened exactly to float64
here; every arithmetic step happens in oracle.c.

Layouts follow the library: q, k, v, o, dout are [B, N, H, d]; lse is [B, H, N].
Definitions cited in oracle.c: "6.2 FlashAttention V2 in depth" sections 5.1
(causal mask), 6.1 (forward and saved logsumexp) and 7 (backward, D vector).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.POINTER(ctypes.c_double)
_PI = ctypes.POINTER(ctypes.c_int64)
_I64 = ctypes.c_int64


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU involved)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_attention_forward.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64,
                                             ctypes.c_int, ctypes.c_double, _P, _P]
    lib.oracle_attention_forward.restype = ctypes.c_int
    lib.oracle_attention_forward_rows.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64,
                                                  ctypes.c_int, ctypes.c_double, _I64,
                                                  _PI, _P, _P]
    lib.oracle_attention_forward_rows.restype = ctypes.c_int
    lib.oracle_attention_backward.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                              ctypes.c_int, ctypes.c_double, _I64, _PI,
                                              _P, _P, _P, _P, _P]
    lib.oracle_attention_backward.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def widen(x) -> np.ndarray:
    """Exact widening to a contiguous float64 array (bf16/fp32 -> fp64 is exact)."""
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


def _shape4(q):
    if q.ndim != 4:
        raise ValueError("expected a [B, N, H, d] tensor")
    B, N, H, d = q.shape
    return int(B), int(N), int(H), int(d)


def attention_forward(q, k, v, causal: bool, scale: float):
    """Full forward pass. Returns (o [B,N,H,d], lse [B,H,N]) as float64 arrays."""
    q, k, v = widen(q), widen(k), widen(v)
    B, N, H, d = _shape4(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, N, H, d] shape")
    o = np.zeros((B, N, H, d), np.float64)
    lse = np.zeros((B, H, N), np.float64)
    rc = _load().oracle_attention_forward(_ptr(q), _ptr(k), _ptr(v), B, H, N, d,
                                          int(bool(causal)), float(scale),
                                          _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_attention_forward failed")
    return o, lse


def attention_forward_rows(q, k, v, causal: bool, scale: float, rows):
    """Forward pass on selected rows. rows: int array [n, 3] of (b, h, i).

    Returns (o_rows [n, d], lse_rows [n]) as float64 arrays.
    """
    q, k, v = widen(q), widen(k), widen(v)
    B, N, H, d = _shape4(q)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    o = np.zeros((n, d), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = _load().oracle_attention_forward_rows(
        _ptr(q), _ptr(k), _ptr(v), B, H, N, d, int(bool(causal)), float(scale), n,
        rows.ctypes.data_as(_PI), _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_attention_forward_rows failed")
    return o, lse


def attention_backward(q, k, v, dout, causal: bool, scale: float, heads=None):
    """Backward pass for selected heads (default: every head, b-major).

    heads: int array [n, 2] of (b, h).  Returns a dict of float64 arrays:
    dq, dk, dv [n, N, d]; lse, D [n, N].
    """
    q, k, v, dout = widen(q), widen(k), widen(v), widen(dout)
    B, N, H, d = _shape4(q)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int64).reshape(-1, 2))
    n = heads.shape[0]
    out = {name: np.zeros((n, N, d), np.float64) for name in ("dq", "dk", "dv")}
    out["lse"] = np.zeros((n, N), np.float64)
    out["D"] = np.zeros((n, N), np.float64)
    rc = _load().oracle_attention_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, int(bool(causal)),
        float(scale), n, heads.ctypes.data_as(_PI), _ptr(out["dq"]), _ptr(out["dk"]),
        _ptr(out["dv"]), _ptr(out["lse"]), _ptr(out["D"]))
    if rc != 0:
        raise RuntimeError("oracle_attention_backward failed")
    return out
