"""ctypes loader for the C oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring). Compiles the C file with
gcc on first use if the shared object is missing, so the CPU test suite works
without a separate build step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_CFLAGS = ["-O2", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11"]

_libs: dict[str, ctypes.CDLL] = {}


def library_path() -> str:
    return _LIB


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``src`` into the shared object ``out`` with gcc."""
    cmd = ["gcc", *_CFLAGS, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load(path: str | None = None) -> ctypes.CDLL:
    path = path or _LIB
    if path in _libs:
        return _libs[path]
    if path == _LIB and not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    f = lib.kda_oracle_prefill
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    f.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, p, p, i64, p, p, ctypes.c_int]
    f.restype = ctypes.c_int
    b = lib.kda_oracle_backward
    b.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, p, p, p, i64, p, p, p, p, p, p, ctypes.c_int]
    b.restype = ctypes.c_int
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def max_threads(lib_path: str | None = None) -> int:
    return int(_load(lib_path).kda_oracle_max_threads())


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, heads=None,
            want_out=True, want_state=True, threads: int = 0, lib_path: str | None = None):
    """Run the fp64 oracle.

    q, k, g: [T, H, K]; v: [T, H, V]; beta: [T, H] (any float dtype; converted to
    fp32, which must already hold the exact values the GPU sees).
    g may also be [T, H]: the scalar-gated delta rule, which is this recurrence with
    the one decay of a token and head applied to every key channel (the Gated
    DeltaNet comparison in tech-noisy.com, "MoE通信とアテンション:MoonEPとFlashKDA").
    cu_seqlens: int [N+1] or None (one sequence). initial_state: [N, H, K, V] or None.
    heads: iterable of head indices to evaluate (default: all).
    Returns (out [T, n_heads, V] float64 or None, final_state [N, n_heads, K, V] float64 or None).
    """
    lib = _load(lib_path)
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    T, H, K = q.shape
    if g.shape == (T, H):
        g = np.ascontiguousarray(np.broadcast_to(g[:, :, None], (T, H, K)))
    V = v.shape[2]
    if k.shape != (T, H, K) or g.shape != (T, H, K) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent input shapes")
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    s0 = None if initial_state is None else _f32(initial_state)
    if s0 is not None and s0.shape != (N, H, K, V):
        raise ValueError("initial_state must be [N, H, K, V]")
    hs = np.arange(H, dtype=np.int64) if heads is None else np.array(list(heads), dtype=np.int64)
    nh = hs.shape[0]
    out = np.empty((T, nh, V), np.float64) if want_out else None
    fs = np.empty((N, nh, K, V), np.float64) if want_state else None
    rc = lib.kda_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), N, T,
                                H, K, V, _ptr(s0), _ptr(hs), nh, _ptr(out), _ptr(fs), int(threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_prefill failed with status {rc}")
    return out, fs


def backward(q, k, v, g, beta, d_out, cu_seqlens=None, initial_state=None, d_final_state=None,
             heads=None, threads: int = 0, lib_path: str | None = None):
    """Gradients of L = sum <d_out, out> + <d_final_state, final_state> (fp64).

    Inputs as :func:`prefill`, plus d_out [T, H, V] and d_final_state [N, H, K, V]
    or None (zero). Returns a dict with dq, dk, dg [T, n_heads, K], dv
    [T, n_heads, V], dbeta [T, n_heads] and d_initial_state [N, n_heads, K, V],
    all float64. For a [T, H] (scalar) gate, dg is [T, n_heads]: the gate is
    applied to every key channel, so its gradient is the sum over the channels.
    """
    lib = _load(lib_path)
    q, k, v, g, beta, d_out = map(_f32, (q, k, v, g, beta, d_out))
    T, H, K = q.shape
    scalar_gate = g.shape == (T, H)
    if scalar_gate:
        g = np.ascontiguousarray(np.broadcast_to(g[:, :, None], (T, H, K)))
    V = v.shape[2]
    if (k.shape != (T, H, K) or g.shape != (T, H, K) or v.shape[:2] != (T, H)
            or beta.shape != (T, H) or d_out.shape != (T, H, V)):
        raise ValueError("inconsistent input shapes")
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    s0 = None if initial_state is None else _f32(initial_state)
    dsT = None if d_final_state is None else _f32(d_final_state)
    for name, a in (("initial_state", s0), ("d_final_state", dsT)):
        if a is not None and a.shape != (N, H, K, V):
            raise ValueError(f"{name} must be [N, H, K, V]")
    hs = np.arange(H, dtype=np.int64) if heads is None else np.array(list(heads), dtype=np.int64)
    nh = hs.shape[0]
    out = dict(dq=np.empty((T, nh, K)), dk=np.empty((T, nh, K)), dv=np.empty((T, nh, V)),
               dg=np.empty((T, nh, K)), dbeta=np.empty((T, nh)),
               d_initial_state=np.empty((N, nh, K, V)))
    rc = lib.kda_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(d_out),
                                 _ptr(cu), N, T, H, K, V, _ptr(s0), _ptr(dsT), _ptr(hs), nh,
                                 _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                 _ptr(out["dbeta"]), _ptr(out["d_initial_state"]), int(threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_backward failed with status {rc}")
    if scalar_gate:
        out["dg"] = out["dg"].sum(axis=2)
    return out
