"""Helpers for GPU parity tests: upload seeded inputs, run the HIP path through the
C ABI, compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import oracle
from linear_attention_04_amd import inputs

# Tolerances per tensor (out and final state separately): bf16 io
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
# fp32 io
F32_MAX_ABS = 1e-5


def torch_mod():
    import torch

    return torch


def to_device(a, bf16: bool):
    torch = torch_mod()
    if a is None:
        return None
    if bf16:
        return torch.from_numpy(inputs.bf16_bits(a)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def to_host(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(x: dict, bf16: bool, packed: bool):
    torch = torch_mod()
    d = {
        "q": to_device(x["q"], bf16),
        "k": to_device(x["k"], bf16),
        "v": to_device(x["v"], bf16),
        "g": to_device(x["g"], False),
        "beta": to_device(x["beta"], False),
        "initial_state": to_device(x.get("initial_state"), False),
        "cu_seqlens": None,
    }
    if packed:
        d["cu_seqlens"] = torch.from_numpy(np.asarray(x["cu_seqlens"], np.int32)).to("cuda")
    return d


def run_gpu(d: dict, final_state=True):
    from linear_attention_04_amd import kda

    torch = torch_mod()
    out, fs = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                                initial_state=d["initial_state"], final_state=final_state)
    torch.cuda.synchronize()
    return out, fs


def run_oracle(x: dict, packed: bool, heads=None):
    return oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                          cu_seqlens=x["cu_seqlens"] if packed else None,
                          initial_state=x.get("initial_state"), heads=heads)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.sqrt(np.sum(ref * ref)))
    rel = float(np.sqrt(np.sum(diff * diff)) / den) if den > 0 else float(np.sqrt(np.sum(diff * diff)))
    return max_abs, rel


def assert_close(name, got, ref, bf16: bool):
    max_abs, rel = errors(got, ref)
    print(f"  {name}: max|err|={max_abs:.3e} relL2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if bf16:
        assert max_abs <= BF16_MAX_ABS, f"{name}: max|err| {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{name}: rel-L2 {rel:.3e} > {BF16_REL_L2}"
    else:
        assert max_abs <= F32_MAX_ABS, f"{name}: max|err| {max_abs:.3e} > {F32_MAX_ABS}"
    return max_abs, rel


def generate_on_device(w, keep_heads, threads: int = 16):
    """Generate ``w`` block by block straight into device tensors (host memory stays
    small for the 131072-token workload); host copies are kept for ``keep_heads``."""
    import concurrent.futures as cf

    torch = torch_mod()
    T, H, K, V = w.total_tokens, w.heads, w.head_k, w.head_v
    io = torch.bfloat16 if w.bf16 else torch.float32
    gshape = (T, H) if w.gate == "scalar" else (T, H, K)
    dev = {
        "q": torch.empty((T, H, K), dtype=io, device="cuda"),
        "k": torch.empty((T, H, K), dtype=io, device="cuda"),
        "v": torch.empty((T, H, V), dtype=io, device="cuda"),
        "g": torch.empty(gshape, dtype=torch.float32, device="cuda"),
        "beta": torch.empty((T, H), dtype=torch.float32, device="cuda"),
    }
    keep = list(keep_heads)
    host = {
        "q": np.empty((T, len(keep), K), np.float32),
        "k": np.empty((T, len(keep), K), np.float32),
        "v": np.empty((T, len(keep), V), np.float32),
        "g": np.empty((T, len(keep)) + gshape[2:], np.float32),
        "beta": np.empty((T, len(keep)), np.float32),
    }

    def work(b):
        blk = inputs.generate_block(w, b)
        t0 = blk["t0"]
        n = blk["q"].shape[0]
        for name in host:
            host[name][t0:t0 + n] = blk[name][:, keep]
        return blk

    with cf.ThreadPoolExecutor(threads) as ex:
        for blk in ex.map(work, range(inputs.num_blocks(w))):
            t0 = blk["t0"]
            n = blk["q"].shape[0]
            for name in dev:
                arr = blk[name]
                if name in ("q", "k", "v") and w.bf16:
                    t = torch.from_numpy(inputs.bf16_bits(arr)).view(torch.bfloat16)
                else:
                    t = torch.from_numpy(arr)
                dev[name][t0:t0 + n].copy_(t)
    s0 = inputs.initial_state(w)
    cu = inputs.cu_seqlens(w)
    dev["initial_state"] = None if s0 is None else torch.from_numpy(s0).to("cuda")
    dev["cu_seqlens"] = torch.from_numpy(cu).to("cuda") if w.num_seqs > 1 else None
    host["initial_state"] = None if s0 is None else np.ascontiguousarray(s0[:, keep])
    host["cu_seqlens"] = cu
    return dev, host


# ---------------------------------------------------------------------------
# backward pass

# Tolerances per gradient tensor (bf16 io), relative to the tensor because the gradients
# span about three decades of magnitude: rel-L2 over the whole tensor, and max|err|
# against the tensor's largest magnitude. Derived from the bf16 rounding model
# (tests/rounding_model.py), which the GPU matches to a few per cent: on the workloads'
# value recipes it predicts rel-L2 1.7e-3 .. 3.6e-3 and max|err| up to 3.8e-3 of the
# largest magnitude for every gradient (pinned in test_rounding_model.py). The bars keep
# 30% over the largest rel-L2 and 2.5x over the largest max|err| (extremes grow with the
# number of elements; the full-size tests see 10^7 of them).
BWD_REL_L2 = 5e-3
BWD_MAX_REL = 1e-2

_ALIGN = 256
_REC_BYTES = 14848
_BREC_BYTES = 12800
_STATE_BYTES = 32768


def _align(x):
    return (x + _ALIGN - 1) // _ALIGN * _ALIGN


def backward_workspace_layout(T, H, N):
    """Byte offsets of the backward workspace areas (bf16, K = V = 128), as the
    library lays them out; tests check the total against kda_backward_workspace_bytes."""
    max_chunks = (T + 15 * N) // 16
    per = max_chunks * H
    off_chunk_seq = _align(4 * (N + 1))
    off_records = off_chunk_seq + _align(4 * max_chunks)
    total = off_records + per * _REC_BYTES
    off_brecords = _align(total)
    off_states = _align(off_brecords + per * _BREC_BYTES)
    off_dstates = _align(off_states + per * _STATE_BYTES)
    return dict(max_chunks=max_chunks, off_states=off_states, off_dstates=off_dstates,
                total=off_dstates + per * _STATE_BYTES)


def decode_state_fragments(raw: np.ndarray) -> np.ndarray:
    """A 128 x 128 bf16 state in fragment layout (32768 bytes) -> [key][value] fp64:
    fragment (ct, ks), lane (c, grp), element e holds value column 16 ct + c and key
    32 ks + 8 grp + e."""
    u16 = np.frombuffer(np.ascontiguousarray(raw).tobytes(), dtype=np.uint16).reshape(8, 4, 64, 8)
    vals = (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = np.empty((128, 128))
    lane = np.arange(64)
    c, grp = lane % 16, lane // 16
    for ct in range(8):
        for ks in range(4):
            for e in range(8):
                key = 32 * ks + 8 * grp + e
                out[key, 16 * ct + c] = vals[ct, ks, :, e]
    return out


def upload_backward(x: dict, d_out, d_fs, packed: bool):
    d = upload(x, True, packed)
    d["d_out"] = to_device(d_out, True)
    d["d_final_state"] = to_device(d_fs, False)
    return d


def run_gpu_backward(d: dict, want_d_initial_state=True, workspace=None):
    from linear_attention_04_amd import kda

    torch = torch_mod()
    r = kda.chunk_prefill_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_out"],
                                   cu_seqlens=d["cu_seqlens"], initial_state=d["initial_state"],
                                   d_final_state=d["d_final_state"],
                                   want_d_initial_state=want_d_initial_state, workspace=workspace)
    torch.cuda.synchronize()
    return r


def run_oracle_backward(x: dict, d_out, d_fs, packed: bool, heads=None):
    return oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_out,
                           cu_seqlens=x["cu_seqlens"] if packed else None,
                           initial_state=x.get("initial_state"), d_final_state=d_fs, heads=heads)


def assert_close_rel(name, got, ref, rel_l2=None, max_rel=None):
    rel_l2 = BWD_REL_L2 if rel_l2 is None else rel_l2
    max_rel = BWD_MAX_REL if max_rel is None else max_rel
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs, rel = errors(got, ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    print(f"  {name}: max|err|={max_abs:.3e} (max|ref|={scale:.3e}) relL2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert rel <= rel_l2, f"{name}: rel-L2 {rel:.3e} > {rel_l2}"
    assert max_abs <= max_rel * max(scale, 1e-30), f"{name}: max|err| {max_abs:.3e} > {max_rel} * {scale:.3e}"
    return max_abs, rel


# The GPU's distance to the oracle against the rounding model's, on the same inputs:
# the model rounds where the kernels round, so the two agree closely (measured: within
# 0.9% over every tensor of the parity tests); the band allows for the fp32 summation
# order and, in small tensors, the few bf16 results that round the other way.
MODEL_BAND = 0.1
MODEL_FLOOR = 2e-4


def assert_model_band(name, got, ref, model):
    """rel-L2 of `got` (GPU) against `ref` (oracle) within MODEL_BAND of the rounding
    model's rel-L2 against the same reference (plus MODEL_FLOOR)."""
    from tests import rounding_model as rm

    e_gpu, e_model = rm.rel_l2(got, ref), rm.rel_l2(model, ref)
    print(f"  {name}: GPU rel-L2 {e_gpu:.3e}, rounding model {e_model:.3e}", flush=True)
    assert abs(e_gpu - e_model) <= MODEL_BAND * e_model + MODEL_FLOOR, \
        f"{name}: GPU rel-L2 {e_gpu:.3e} outside the rounding model's {e_model:.3e} +- {MODEL_BAND:.0%}"


def first_heads(x: dict, n: int) -> dict:
    """The inputs of heads 0 .. n - 1 only (head is axis 1 of every per-head array)."""
    out = dict(x)
    for key in ("q", "k", "v", "g", "beta", "initial_state"):
        if x.get(key) is not None:
            out[key] = np.ascontiguousarray(x[key][:, :n])
    return out


def dg_term_scale(x: dict, ref: dict, chunk: int = 16) -> np.ndarray:
    """Per-element magnitude of the products dg is summed from, shaped like dg.

    Inside a chunk the gradient reaching the running gate is, per token and channel,
    dG_r = q_r dq_r + k_r dk_r - 2 (K~_r dK~_r + K^d_r dK^d_r) (every gated factor
    is q or k times an exponential of G, and dq, dk collect the same products), and
    dg_t is the sum of dG_r over the chunk's tokens r >= t. Rounding errors of dg
    therefore scale with these products, not with dg itself, which can be many
    times smaller (strong decays, beta = 1 with unit keys). Returns the in-chunk
    suffix sums of |q dq| + |k dk| (summed over the channels for a scalar gate)."""
    q, k = np.asarray(x["q"], np.float64), np.asarray(x["k"], np.float64)
    m = np.abs(q * ref["dq"]) + np.abs(k * ref["dk"])
    cu = np.asarray(x["cu_seqlens"]) if x.get("cu_seqlens") is not None and len(x["cu_seqlens"]) > 2 \
        else np.array([0, q.shape[0]])
    out = np.zeros_like(m)
    for n in range(len(cu) - 1):
        for c0 in range(int(cu[n]), int(cu[n + 1]), chunk):
            c1 = min(c0 + chunk, int(cu[n + 1]))
            out[c0:c1] = np.cumsum(m[c0:c1][::-1], axis=0)[::-1]
    if np.ndim(x["g"]) == 2:
        out = out.sum(axis=-1)
    return out


def assert_dg_close(got, ref_dg, scale, rel_l2=None, max_rel=None):
    """dg against the oracle, relative to |dg| plus the magnitude of the products it is
    summed from (dg_term_scale): the same bars as the other gradients, rel-L2 and
    max|err| against max(|dg| + scale)."""
    rel_l2 = BWD_REL_L2 if rel_l2 is None else rel_l2
    max_rel = BWD_MAX_REL if max_rel is None else max_rel
    got = np.asarray(got, np.float64)
    ref_dg = np.asarray(ref_dg, np.float64)
    diff = got - ref_dg
    den = float(np.linalg.norm(ref_dg) + np.linalg.norm(scale))
    rel = float(np.linalg.norm(diff)) / max(den, 1e-300)
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    top = float(np.max(np.abs(ref_dg) + scale)) if diff.size else 0.0
    print(f"  dg: max|err|={max_abs:.3e} (max|dg|+scale={top:.3e}) rel-L2 against |dg|+scale={rel:.3e}",
          flush=True)
    assert np.all(np.isfinite(got)), "dg: non-finite values"
    assert rel <= rel_l2, f"dg: rel-L2 {rel:.3e} > {rel_l2}"
    assert max_abs <= max_rel * max(top, 1e-30), f"dg: max|err| {max_abs:.3e} > {max_rel} * {top:.3e}"
