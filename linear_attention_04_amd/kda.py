"""Python binding of libkda.so (include/kda.h).

The functions named like the C entry points take raw device pointers (ints) and a
``KdaDims``; :func:`chunk_prefill` is the torch-facing convenience wrapper that
allocates outputs and workspace with torch and passes torch's current stream.
Both only marshal arguments: every step of the computation runs in the HIP
kernels of libkda.so, and there is no fallback when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_IO_BF16 = 0
KDA_IO_F32 = 1
KDA_GATE_CHANNEL = 0
KDA_GATE_SCALAR = 1
KDA_OK = 0
KDA_ERR_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_ALIGN = -3
KDA_ERR_WORKSPACE = -4
KDA_ERR_LAUNCH = -5
KDA_ERR_CAPACITY = -6
KDA_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = (
    "kda_workspace_bytes",
    "kda_chunk_prefill",
    "kda_chunk_prefill_fused",
    "kda_intra_chunk",
    "kda_inter_chunk",
    "kda_decode_step",
    "kda_backward_workspace_bytes",
    "kda_chunk_prefill_backward",
    "kda_chunk_prefill_for_backward",
    "kda_backward_records",
    "kda_backward_states",
    "kda_backward_state_grad",
    "kda_backward_token_grad",
    "kda_check_seqlens",
    "kda_chunk_prefill_noalloc",
    "kda_status_string",
    "kda_version",
)


class KdaDims(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("num_heads", ctypes.c_int32),
        ("head_k", ctypes.c_int32),
        ("head_v", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("gate_kind", ctypes.c_int32),
    ]


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kda_status_string(status)} (status {status})")
        self.status = status


_lib = None
_lib_path = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libkda.so (from `path`, else the in-tree build), or return the library
    already loaded; raises if it has not been built, or if `path` names a library other
    than the one already loaded (one process holds one copy of the kernels).

    torch is imported first. The buffers and streams the library works on come from
    torch, so the library must bind to the HIP runtime torch has loaded. Loaded before
    torch, it would bring in the system ROCm's runtime instead, a second runtime in the
    process, and its launches on torch's streams fail."""
    global _lib, _lib_path
    if _lib is not None:
        if path is not None and os.path.realpath(path) != _lib_path:
            raise RuntimeError(f"libkda is already loaded from {_lib_path}; cannot also load {path}")
        return _lib
    path = LIB_PATH if path is None else path
    real = os.path.realpath(path)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m linear_attention_04_amd.build`")
    import torch  # noqa: F401  (its HIP runtime first)

    lib = ctypes.CDLL(real)
    p, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dims_p = ctypes.POINTER(KdaDims)
    lib.kda_workspace_bytes.argtypes = [dims_p]
    lib.kda_workspace_bytes.restype = sz
    lib.kda_chunk_prefill.argtypes = [p, p, p, p, p, p, p, p, p, dims_p, p, sz, p]
    lib.kda_chunk_prefill.restype = i32
    lib.kda_chunk_prefill_fused.argtypes = [p, p, p, p, p, p, p, p, p, dims_p, p, sz, p]
    lib.kda_chunk_prefill_fused.restype = i32
    lib.kda_intra_chunk.argtypes = [p, p, p, p, p, dims_p, p, sz, p]
    lib.kda_intra_chunk.restype = i32
    lib.kda_inter_chunk.argtypes = [p, p, p, p, p, dims_p, p, sz, p]
    lib.kda_inter_chunk.restype = i32
    lib.kda_decode_step.argtypes = [p, p, p, p, p, p, p, dims_p, p]
    lib.kda_decode_step.restype = i32
    lib.kda_backward_workspace_bytes.argtypes = [dims_p]
    lib.kda_backward_workspace_bytes.restype = sz
    lib.kda_chunk_prefill_backward.argtypes = [p] * 15 + [dims_p, p, sz, p]
    lib.kda_chunk_prefill_backward.restype = i32
    lib.kda_chunk_prefill_for_backward.argtypes = [p, p, p, p, p, p, p, p, p, dims_p, p, sz, p]
    lib.kda_chunk_prefill_for_backward.restype = i32
    lib.kda_backward_records.argtypes = [p] * 5 + [dims_p, p, sz, p]
    lib.kda_backward_records.restype = i32
    lib.kda_backward_states.argtypes = [p] * 3 + [dims_p, p, sz, p]
    lib.kda_backward_states.restype = i32
    lib.kda_backward_state_grad.argtypes = [p] * 4 + [dims_p, p, sz, p]
    lib.kda_backward_state_grad.restype = i32
    lib.kda_backward_token_grad.argtypes = [p] * 12 + [dims_p, p, sz, p]
    lib.kda_backward_token_grad.restype = i32
    lib.kda_chunk_prefill_noalloc.argtypes = [p, p, p, p, p, p, p, p, p, dims_p, p]
    lib.kda_chunk_prefill_noalloc.restype = i32
    lib.kda_check_seqlens.argtypes = [p, ctypes.c_int32, ctypes.c_int64, p, p]
    lib.kda_check_seqlens.restype = i32
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = i32
    _lib = lib
    _lib_path = real
    return lib


def kda_workspace_bytes(dims: KdaDims) -> int:
    return int(load_library().kda_workspace_bytes(ctypes.byref(dims)))


def kda_chunk_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, dims: KdaDims,
                      workspace, workspace_bytes: int, stream) -> int:
    return int(load_library().kda_chunk_prefill(q, k, v, g, beta, cu_seqlens, initial_state, out,
                                                final_state, ctypes.byref(dims), workspace,
                                                workspace_bytes, stream))


def kda_chunk_prefill_fused(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, dims: KdaDims,
                            workspace, workspace_bytes: int, stream) -> int:
    return int(load_library().kda_chunk_prefill_fused(q, k, v, g, beta, cu_seqlens, initial_state, out,
                                                      final_state, ctypes.byref(dims), workspace,
                                                      workspace_bytes, stream))


def kda_intra_chunk(q, k, g, beta, cu_seqlens, dims: KdaDims, workspace, workspace_bytes: int,
                    stream) -> int:
    return int(load_library().kda_intra_chunk(q, k, g, beta, cu_seqlens, ctypes.byref(dims),
                                              workspace, workspace_bytes, stream))


def kda_inter_chunk(v, cu_seqlens, initial_state, out, final_state, dims: KdaDims, workspace,
                    workspace_bytes: int, stream) -> int:
    return int(load_library().kda_inter_chunk(v, cu_seqlens, initial_state, out, final_state,
                                              ctypes.byref(dims), workspace, workspace_bytes, stream))


def kda_decode_step(q, k, v, g, beta, state, out, dims: KdaDims, stream) -> int:
    return int(load_library().kda_decode_step(q, k, v, g, beta, state, out, ctypes.byref(dims), stream))


def kda_backward_workspace_bytes(dims: KdaDims) -> int:
    return int(load_library().kda_backward_workspace_bytes(ctypes.byref(dims)))


def kda_chunk_prefill_backward(q, k, v, g, beta, cu_seqlens, initial_state, d_out, d_final_state, dq, dk, dv,
                               dg, dbeta, d_initial_state, dims: KdaDims, workspace, workspace_bytes: int,
                               stream) -> int:
    return int(load_library().kda_chunk_prefill_backward(q, k, v, g, beta, cu_seqlens, initial_state, d_out,
                                                         d_final_state, dq, dk, dv, dg, dbeta, d_initial_state,
                                                         ctypes.byref(dims), workspace, workspace_bytes,
                                                         stream))


def kda_chunk_prefill_for_backward(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                                   dims: KdaDims, workspace, workspace_bytes: int, stream) -> int:
    return int(load_library().kda_chunk_prefill_for_backward(q, k, v, g, beta, cu_seqlens, initial_state, out,
                                                             final_state, ctypes.byref(dims), workspace,
                                                             workspace_bytes, stream))


def kda_backward_records(q, k, g, beta, cu_seqlens, dims: KdaDims, workspace, workspace_bytes: int,
                         stream) -> int:
    return int(load_library().kda_backward_records(q, k, g, beta, cu_seqlens, ctypes.byref(dims), workspace,
                                                   workspace_bytes, stream))


def kda_backward_states(v, cu_seqlens, initial_state, dims: KdaDims, workspace, workspace_bytes: int,
                        stream) -> int:
    return int(load_library().kda_backward_states(v, cu_seqlens, initial_state, ctypes.byref(dims), workspace,
                                                  workspace_bytes, stream))


def kda_backward_state_grad(d_out, cu_seqlens, d_final_state, d_initial_state, dims: KdaDims, workspace,
                            workspace_bytes: int, stream) -> int:
    return int(load_library().kda_backward_state_grad(d_out, cu_seqlens, d_final_state, d_initial_state,
                                                      ctypes.byref(dims), workspace, workspace_bytes, stream))


def kda_backward_token_grad(q, k, v, g, beta, d_out, cu_seqlens, dq, dk, dv, dg, dbeta, dims: KdaDims,
                            workspace, workspace_bytes: int, stream) -> int:
    return int(load_library().kda_backward_token_grad(q, k, v, g, beta, d_out, cu_seqlens, dq, dk, dv, dg, dbeta,
                                                      ctypes.byref(dims), workspace, workspace_bytes, stream))


def kda_chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, dims: KdaDims,
                              stream) -> int:
    return int(load_library().kda_chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, initial_state, out,
                                                        final_state, ctypes.byref(dims), stream))


def kda_check_seqlens(cu_seqlens, num_seqs: int, total_tokens: int, result, stream) -> int:
    return int(load_library().kda_check_seqlens(cu_seqlens, num_seqs, total_tokens, result, stream))


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def kda_version() -> int:
    return int(load_library().kda_version())


# ---------------------------------------------------------------------------
# torch-facing wrapper
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _nbytes(t):
    return t.numel() * t.element_size()


def make_dims(q, v, cu_seqlens=None, g=None) -> KdaDims:
    """Sizes from the tensors; a g of shape [T, H] selects the scalar gate."""
    import torch

    T, H, K = q.shape
    V = v.shape[2]
    io = KDA_IO_BF16 if q.dtype == torch.bfloat16 else KDA_IO_F32
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    gate = KDA_GATE_SCALAR if (g is not None and g.dim() == 2) else KDA_GATE_CHANNEL
    return KdaDims(T, H, K, V, N, io, gate)


def workspace_for(dims: KdaDims, device):
    import torch

    nbytes = kda_workspace_bytes(dims)
    if nbytes == 0:
        raise KdaError(KDA_ERR_UNSUPPORTED, "kda_workspace_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _check_tensors(q, k, v, g, beta, cu_seqlens, initial_state):
    import torch

    io = q.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    for name, t, dt in (("k", k, io), ("v", v, io), ("g", g, torch.float32), ("beta", beta, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if initial_state is not None and initial_state.dtype != torch.float32:
        raise TypeError("initial_state must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("cu_seqlens", cu_seqlens),
                    ("initial_state", initial_state)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k must be [T, H, K] and v [T, H, V]")
    T, H, K = q.shape
    if k.shape != (T, H, K) or g.shape not in ((T, H, K), (T, H)) or v.shape[:2] != (T, H) \
            or beta.shape != (T, H):
        raise ValueError("shape mismatch: q, k [T,H,K], g [T,H,K] or [T,H], v [T,H,V], beta [T,H]")
    if cu_seqlens is not None and (cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2):
        raise ValueError("cu_seqlens must be int32 [N + 1] with N >= 1")
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta), ("cu_seqlens", cu_seqlens),
                    ("initial_state", initial_state)):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if initial_state is not None:
        N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
        if tuple(initial_state.shape) != (N, H, K, v.shape[2]):
            raise ValueError(f"initial_state must be [N, H, K, V] = {(N, H, K, v.shape[2])}, "
                             f"got {tuple(initial_state.shape)}")


def _check_outputs(v, dims, out, final_state):
    """Caller-supplied output buffers: the C ABI cannot see their sizes, so a short one
    would be written past its end. Checked before anything is launched."""
    import torch

    if out is not None:
        if out.dtype != v.dtype or tuple(out.shape) != tuple(v.shape) or not out.is_cuda \
                or not out.is_contiguous() or out.device != v.device:
            raise ValueError(f"out must be a contiguous {v.dtype} tensor {tuple(v.shape)} on {v.device}")
    if final_state is not None and final_state is not True:
        want = (dims.num_seqs, dims.num_heads, dims.head_k, dims.head_v)
        if final_state.dtype != torch.float32 or tuple(final_state.shape) != want or not final_state.is_cuda \
                or not final_state.is_contiguous() or final_state.device != v.device:
            raise ValueError(f"final_state must be a contiguous float32 tensor {want} on {v.device}")


def chunk_prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, out=None,
                  final_state=True, workspace=None, stream=None, fused=False):
    """Chunked KDA prefill on the current device.

    q, k: [T, H, K]; v: [T, H, V] (bf16 or fp32); beta: [T, H] fp32;
    g: [T, H, K] fp32 (per-channel gate) or [T, H] fp32 (scalar gate, Gated DeltaNet);
    cu_seqlens: int32 [N+1] or None; initial_state: [N, H, K, V] fp32 or None.
    final_state: True to allocate and return it, a tensor to write into, or None.
    fused: run the single-kernel form (kda_chunk_prefill_fused; bf16 only).
    Returns (out, final_state).
    """
    import torch

    _check_tensors(q, k, v, g, beta, cu_seqlens, initial_state)
    dims = make_dims(q, v, cu_seqlens, g)
    _check_outputs(v, dims, out, final_state)
    if workspace is None:
        workspace = workspace_for(dims, q.device)
    elif _nbytes(workspace) < kda_workspace_bytes(dims) or not workspace.is_cuda or not workspace.is_contiguous() \
            or workspace.device != q.device:
        raise ValueError(f"workspace must be a contiguous buffer of at least {kda_workspace_bytes(dims)} bytes "
                         f"on {q.device}")
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    if final_state is True:
        final_state = torch.empty((dims.num_seqs, dims.num_heads, dims.head_k, dims.head_v),
                                  dtype=torch.float32, device=q.device)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    entry = kda_chunk_prefill_fused if fused else kda_chunk_prefill
    st = entry(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(initial_state),
               _ptr(out), _ptr(final_state), dims, _ptr(workspace), _nbytes(workspace), s)
    if st != KDA_OK:
        raise KdaError(st, entry.__name__)
    return out, final_state


def decode_step(q, k, v, g, beta, state, out=None, stream=None):
    """One decode step for B sequences: q, k [B, H, K], v [B, H, V] (bf16 or fp32),
    g [B, H, K] or [B, H] fp32, beta [B, H] fp32, state [B, H, K, V] fp32 (updated in
    place). Returns out [B, H, V]."""
    import torch

    io = q.dtype
    B, H, K = q.shape
    V = v.shape[2]
    for name, t, dt in (("k", k, io), ("v", v, io), ("g", g, torch.float32), ("beta", beta, torch.float32),
                        ("state", state, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if k.shape != (B, H, K) or v.shape[:2] != (B, H) or g.shape not in ((B, H, K), (B, H)) \
            or beta.shape != (B, H) or state.shape != (B, H, K, V):
        raise ValueError("shape mismatch: q, k [B,H,K], v [B,H,V], g [B,H,K] or [B,H], beta [B,H], "
                         "state [B,H,K,V]")
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    dims = KdaDims(B, H, K, V, B, KDA_IO_BF16 if io == torch.bfloat16 else KDA_IO_F32,
                   KDA_GATE_SCALAR if g.dim() == 2 else KDA_GATE_CHANNEL)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    st = kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out), dims, s)
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step")
    return out


def check_seqlens(cu_seqlens, total_tokens: int) -> int:
    """Checks packed-sequence boundaries (int32 [N + 1] on the device) for
    cu[0] = 0, non-decreasing, cu[N] = total_tokens, on the current stream. Returns -1
    if they hold, else the first index at which one fails (waits for the result)."""
    import torch

    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous() \
            or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2:
        raise ValueError("cu_seqlens must be a contiguous int32 device tensor of N + 1 >= 2 entries")
    result = torch.empty(1, dtype=torch.int32, device=cu_seqlens.device)
    s = torch.cuda.current_stream(cu_seqlens.device).cuda_stream
    st = kda_check_seqlens(_ptr(cu_seqlens), cu_seqlens.shape[0] - 1, int(total_tokens), _ptr(result), s)
    if st != KDA_OK:
        raise KdaError(st, "kda_check_seqlens")
    return int(result.item())


def _check_d_out(v, d_out, d_final_state, dims):
    import torch

    if d_out.dtype != v.dtype or d_out.shape != v.shape or not d_out.is_cuda or not d_out.is_contiguous():
        raise ValueError("d_out must be a contiguous device tensor like v")
    if d_final_state is not None:
        want = (dims.num_seqs, dims.num_heads, dims.head_k, dims.head_v)
        if d_final_state.dtype != torch.float32 or tuple(d_final_state.shape) != want \
                or not d_final_state.is_cuda or not d_final_state.is_contiguous():
            raise ValueError("d_final_state must be a contiguous fp32 device tensor [N, H, K, V]")


def _backward_workspace(dims, device, workspace, allocate=True):
    """The caller's backward workspace, checked, or (allocate=True) a new one."""
    import torch

    nbytes = kda_backward_workspace_bytes(dims)
    if nbytes == 0:
        raise KdaError(KDA_ERR_UNSUPPORTED, "kda_backward_workspace_bytes")
    if workspace is None:
        if not allocate:
            raise ValueError("workspace is required: pass the one chunk_prefill_for_backward filled")
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if _nbytes(workspace) < nbytes or not workspace.is_cuda or not workspace.is_contiguous() \
            or workspace.device != torch.device(device):
        raise ValueError(f"workspace must be a contiguous buffer of at least {nbytes} bytes on {device}")
    return workspace


def _gradient_buffers(q, k, v, g, beta, dims, want_d_initial_state):
    import torch

    return dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
                d_initial_state=torch.empty((dims.num_seqs, dims.num_heads, dims.head_k, dims.head_v),
                                            dtype=torch.float32, device=q.device)
                if want_d_initial_state else None)


def chunk_prefill_backward(q, k, v, g, beta, d_out, cu_seqlens=None, initial_state=None, d_final_state=None,
                           want_d_initial_state=True, workspace=None, stream=None):
    """Gradients of chunk_prefill (bf16, K = V = 128) for L = <d_out, out> +
    <d_final_state, final_state>.

    Inputs as :func:`chunk_prefill`, plus d_out [T, H, V] bf16 and d_final_state
    [N, H, K, V] fp32 or None. Returns a dict: dq, dk [T, H, K] and dv [T, H, V] bf16,
    dg fp32 shaped like g, dbeta [T, H] fp32, d_initial_state [N, H, K, V] fp32 (or
    None when want_d_initial_state is False).
    """
    import torch

    _check_tensors(q, k, v, g, beta, cu_seqlens, initial_state)
    dims = make_dims(q, v, cu_seqlens, g)
    _check_d_out(v, d_out, d_final_state, dims)
    workspace = _backward_workspace(dims, q.device, workspace)
    out = _gradient_buffers(q, k, v, g, beta, dims, want_d_initial_state)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    st = kda_chunk_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                    _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), _ptr(out["dq"]),
                                    _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                                    _ptr(out["d_initial_state"]), dims, _ptr(workspace), _nbytes(workspace), s)
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_prefill_backward")
    return out


def chunk_prefill_for_backward(q, k, v, g, beta, cu_seqlens=None, initial_state=None, out=None,
                               final_state=True, workspace=None, stream=None):
    """The forward of a training step (kda_chunk_prefill_for_backward): as
    :func:`chunk_prefill` (bf16, K = V = 128), and the backward workspace it fills.
    Returns (out, final_state, workspace); pass the workspace, untouched, to
    :func:`chunk_prefill_backward_from_saved` with the same inputs."""
    import torch

    _check_tensors(q, k, v, g, beta, cu_seqlens, initial_state)
    dims = make_dims(q, v, cu_seqlens, g)
    _check_outputs(v, dims, out, final_state)
    workspace = _backward_workspace(dims, q.device, workspace)
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    if final_state is True:
        final_state = torch.empty((dims.num_seqs, dims.num_heads, dims.head_k, dims.head_v),
                                  dtype=torch.float32, device=q.device)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    st = kda_chunk_prefill_for_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                        _ptr(initial_state), _ptr(out), _ptr(final_state), dims,
                                        _ptr(workspace), _nbytes(workspace), s)
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_prefill_for_backward")
    return out, final_state, workspace


def chunk_prefill_backward_from_saved(q, k, v, g, beta, d_out, workspace, cu_seqlens=None,
                                      d_final_state=None, want_d_initial_state=True, stream=None):
    """The backward of a training step whose forward was
    :func:`chunk_prefill_for_backward` on these inputs and `workspace`: only the
    reverse pass and the token gradients run (kda_backward_state_grad, then
    kda_backward_token_grad). Returns the gradients as :func:`chunk_prefill_backward`."""
    import torch

    _check_tensors(q, k, v, g, beta, cu_seqlens, initial_state=None)
    dims = make_dims(q, v, cu_seqlens, g)
    _check_d_out(v, d_out, d_final_state, dims)
    # the reverse pass reads the records and chunk states the training forward left in
    # this workspace: a fresh buffer would hold none of them
    workspace = _backward_workspace(dims, q.device, workspace, allocate=False)
    out = _gradient_buffers(q, k, v, g, beta, dims, want_d_initial_state)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else stream
    st = kda_backward_state_grad(_ptr(d_out), _ptr(cu_seqlens), _ptr(d_final_state), _ptr(out["d_initial_state"]),
                                 dims, _ptr(workspace), _nbytes(workspace), s)
    if st != KDA_OK:
        raise KdaError(st, "kda_backward_state_grad")
    st = kda_backward_token_grad(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(d_out), _ptr(cu_seqlens),
                                 _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                 _ptr(out["dbeta"]), dims, _ptr(workspace), _nbytes(workspace), s)
    if st != KDA_OK:
        raise KdaError(st, "kda_backward_token_grad")
    return out


_CHUNK_KDA_FN = None


def _chunk_kda_function():
    """The torch.autograd.Function behind :func:`chunk_kda`, made on first use (the
    module itself imports torch only when a torch-facing function runs)."""
    global _CHUNK_KDA_FN
    if _CHUNK_KDA_FN is not None:
        return _CHUNK_KDA_FN
    import torch

    class ChunkKDA(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, g, beta, cu_seqlens, initial_state):
            out, final_state, ws = chunk_prefill_for_backward(q, k, v, g, beta, cu_seqlens=cu_seqlens,
                                                              initial_state=initial_state)
            ctx.save_for_backward(q, k, v, g, beta, cu_seqlens, ws)
            ctx.has_initial_state = initial_state is not None
            ctx.set_materialize_grads(False)  # an output outside the loss arrives as None
            return out, final_state

        @staticmethod
        def backward(ctx, d_out, d_final_state):
            q, k, v, g, beta, cu_seqlens, ws = ctx.saved_tensors
            d_out = torch.zeros_like(v) if d_out is None else d_out.to(v.dtype).contiguous()
            if d_final_state is not None:
                d_final_state = d_final_state.to(torch.float32).contiguous()
            want_ds0 = ctx.has_initial_state and ctx.needs_input_grad[6]
            grads = chunk_prefill_backward_from_saved(q, k, v, g, beta, d_out, ws, cu_seqlens=cu_seqlens,
                                                      d_final_state=d_final_state,
                                                      want_d_initial_state=want_ds0)
            return (grads["dq"], grads["dk"], grads["dv"], grads["dg"], grads["dbeta"], None,
                    grads["d_initial_state"] if want_ds0 else None)

    _CHUNK_KDA_FN = ChunkKDA
    return ChunkKDA


def chunk_kda(q, k, v, g, beta, cu_seqlens=None, initial_state=None, output_final_state=True):
    """Chunked KDA prefill with torch autograd: returns (out, final_state or None).

    Arguments as :func:`chunk_prefill`. When gradients are wanted (grad mode on and
    any of q, k, v, g, beta, initial_state requiring them), the forward runs
    kda_chunk_prefill_for_backward and keeps its backward workspace on the autograd
    graph; backward() then runs only the reverse pass and the token gradients
    (:func:`chunk_prefill_backward_from_saved`) and returns dq, dk, dv (bf16), dg,
    dbeta and the initial state's gradient (fp32). That path is bf16 with K = V = 128;
    other inputs raise KdaError. Otherwise this is :func:`chunk_prefill`.
    """
    import torch

    inputs = (q, k, v, g, beta, initial_state)
    if torch.is_grad_enabled() and any(t is not None and t.requires_grad for t in inputs):
        out, final_state = _chunk_kda_function().apply(q, k, v, g, beta, cu_seqlens, initial_state)
    else:
        out, final_state = chunk_prefill(q, k, v, g, beta, cu_seqlens=cu_seqlens, initial_state=initial_state,
                                         final_state=True if output_final_state else None)
    return out, (final_state if output_final_state else None)
