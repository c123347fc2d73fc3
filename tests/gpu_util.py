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
