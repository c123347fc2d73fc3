"""Seeded synthetic inputs for KDA prefill workloads.

This module only draws random numbers and shapes them into the tensors a KDA
prefill call takes. It holds none of the method's arithmetic, so both the GPU
path and the fp64 oracle can be fed from it without sharing any computation.

Workloads follow the shapes the FlashKDA benchmark discussion uses
(tech-noisy.com, "MoE通信とアテンション:MoonEPとFlashKDA": T=8192, head
dimension 128, H in {64, 96}, fixed and variable length, K=V=128 only) plus a
tiny fp32 case and a long-context case. The pages publish no dataset or length
mix, so every input here is synthetic:

* q, k ~ N(0, 1) per element, then L2-normalised over the key dimension; q is
  additionally scaled by 1/sqrt(K) (the kernel applies no scale of its own).
* v ~ N(0, 1).
* beta = sigmoid(N(0, 1)), one scalar per token and head.
* g = -s * softplus(N(0, 1)), one log-decay per token, head and key channel
  (s = 0.1, or 0.02 for the long-context case); scalar-gate workloads (the
  Gated DeltaNet comparison of that benchmark discussion) draw one per token and
  head instead.
* For bf16 workloads q, k and v are rounded to bf16 (round to nearest even);
  g, beta and the states stay fp32.
* Initial states, where a workload has one, are 0.02 * N(0, 1) in fp32.
* Backward passes receive d_out ~ N(0, 1) (bf16-exact for bf16 workloads) and a
  final-state gradient 0.02 * N(0, 1) in fp32, from a stream of their own
  (:func:`output_gradients`).

Random numbers are drawn block by block over 1024-token blocks with
``numpy.random.default_rng([seed, block])`` in the order q, k, v, beta, g, so a
block can be regenerated on its own (used for the 131072-token case).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

BLOCK_TOKENS = 1024
_STATE_STREAM = 10**6
_LENGTH_STREAM = 10**6 + 1
_GRAD_STREAM = 10**6 + 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic KDA prefill workload."""

    name: str
    seed: int
    heads: int
    total_tokens: int
    head_k: int
    head_v: int
    io_dtype: str  # "bf16" or "f32": dtype of q, k, v and out
    gate_scale: float
    has_initial_state: bool
    num_seqs: int = 1
    lengths: tuple | None = None  # explicit sequence lengths (else drawn, see seq_lengths)
    gate: str = "channel"  # "channel": g [T, H, K]; "scalar": g [T, H]

    @property
    def bf16(self) -> bool:
        return self.io_dtype == "bf16"


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_f32_h2_t64_d16", 0, 2, 64, 16, 16, "f32", 0.1, False),
        Workload("fixed_h64_t8192", 1, 64, 8192, 128, 128, "bf16", 0.1, False),
        Workload("fixed_h96_t8192_s0", 2, 96, 8192, 128, 128, "bf16", 0.1, True),
        Workload("varlen_h96_t8192_n8", 3, 96, 8192, 128, 128, "bf16", 0.1, False, num_seqs=8),
        Workload("long_h64_t131072_s0", 4, 64, 131072, 128, 128, "bf16", 0.02, True),
    )
}


def custom_workload(name: str, seed: int, heads: int, total_tokens: int | None = None,
                    head_k: int = 128, head_v: int = 128, io_dtype: str = "bf16",
                    gate_scale: float = 0.1, has_initial_state: bool = False, num_seqs: int = 1,
                    lengths=None, gate: str = "channel") -> Workload:
    """A workload with the standard value recipe at other sizes (parity tests).
    ``lengths`` fixes the packed sequence lengths (total_tokens and num_seqs follow)."""
    if lengths is not None:
        lengths = tuple(int(n) for n in lengths)
        total_tokens, num_seqs = sum(lengths), len(lengths)
    return Workload(name, seed, heads, total_tokens, head_k, head_v, io_dtype, gate_scale,
                    has_initial_state, num_seqs, lengths, gate)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding the bf16 value."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (int16) of fp32 values that are already exact bf16 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16).view(np.int16)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def generate_block(w: Workload, block: int) -> dict:
    """Tokens [block*1024, ...) of workload ``w`` (all heads)."""
    t0 = block * BLOCK_TOKENS
    tb = min(BLOCK_TOKENS, w.total_tokens - t0)
    if tb <= 0:
        raise ValueError("block out of range")
    rng = np.random.default_rng([w.seed, block])
    H, K, V = w.heads, w.head_k, w.head_v
    q = rng.standard_normal((tb, H, K), dtype=np.float32)
    k = rng.standard_normal((tb, H, K), dtype=np.float32)
    v = rng.standard_normal((tb, H, V), dtype=np.float32)
    beta = rng.standard_normal((tb, H), dtype=np.float32)
    g = rng.standard_normal((tb, H) if w.gate == "scalar" else (tb, H, K), dtype=np.float32)
    q = _unit_rows(q) * np.float32(1.0 / np.sqrt(K))
    k = _unit_rows(k)
    beta = _sigmoid(beta)
    g = (np.float32(-w.gate_scale) * _softplus(g)).astype(np.float32)
    if w.bf16:
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return {"t0": t0, "q": q, "k": k, "v": v, "g": g, "beta": beta}


def num_blocks(w: Workload) -> int:
    return (w.total_tokens + BLOCK_TOKENS - 1) // BLOCK_TOKENS


def seq_lengths(w: Workload) -> np.ndarray:
    """Per-sequence lengths. Several sequences: cut points drawn uniformly without
    replacement, redrawn until every length is >= 64 and none is a multiple of 16."""
    if w.lengths is not None:
        return np.array(w.lengths, dtype=np.int64)
    if w.num_seqs == 1:
        return np.array([w.total_tokens], dtype=np.int64)
    rng = np.random.default_rng([w.seed, _LENGTH_STREAM])
    T, N = w.total_tokens, w.num_seqs
    min_len = min(64, max(1, T // (2 * N)))
    for _ in range(100000):
        cuts = np.sort(rng.choice(np.arange(1, T), size=N - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [T]]))
        if np.all(lens >= min_len) and (T // N < 16 or np.all(lens % 16 != 0)):
            return lens.astype(np.int64)
    raise RuntimeError("could not draw sequence lengths")


def cu_seqlens(w: Workload) -> np.ndarray:
    lens = seq_lengths(w)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def initial_state(w: Workload) -> np.ndarray | None:
    if not w.has_initial_state:
        return None
    rng = np.random.default_rng([w.seed, _STATE_STREAM])
    s = rng.standard_normal((w.num_seqs, w.heads, w.head_k, w.head_v), dtype=np.float32)
    return (np.float32(0.02) * s).astype(np.float32)


def output_gradients(w: Workload) -> tuple:
    """(d_out [T, H, V], d_final_state [N, H, K, V]) fp32, the gradients a backward pass
    of ``w`` receives; d_out holds bf16-exact values for bf16 workloads."""
    rng = np.random.default_rng([w.seed, _GRAD_STREAM])
    T, H, K, V = w.total_tokens, w.heads, w.head_k, w.head_v
    d_out = rng.standard_normal((T, H, V), dtype=np.float32)
    if w.bf16:
        d_out = round_to_bf16(d_out)
    d_fs = (np.float32(0.02) * rng.standard_normal((w.num_seqs, H, K, V), dtype=np.float32)).astype(np.float32)
    return d_out, d_fs


def generate(w: Workload, threads: int | None = None) -> dict:
    """All inputs of ``w`` as fp32 numpy arrays (bf16-exact values for bf16 workloads).

    Keys: q, k, v [T,H,K|V]; g [T,H,K] ([T,H] for a scalar gate); beta [T,H]; cu_seqlens int32[N+1];
    initial_state [N,H,K,V] or None.
    """
    nb = num_blocks(w)
    T, H, K, V = w.total_tokens, w.heads, w.head_k, w.head_v
    out = {
        "q": np.empty((T, H, K), np.float32),
        "k": np.empty((T, H, K), np.float32),
        "v": np.empty((T, H, V), np.float32),
        "g": np.empty((T, H) if w.gate == "scalar" else (T, H, K), np.float32),
        "beta": np.empty((T, H), np.float32),
    }

    def fill(b):
        blk = generate_block(w, b)
        t0 = blk["t0"]
        for name in ("q", "k", "v", "g", "beta"):
            arr = blk[name]
            out[name][t0:t0 + arr.shape[0]] = arr
        return b

    workers = threads or min(nb, max(1, (os.cpu_count() or 1)), 16)
    if nb == 1 or workers == 1:
        for b in range(nb):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nb)))
    out["cu_seqlens"] = cu_seqlens(w)
    out["initial_state"] = initial_state(w)
    return out


def algorithmic_counts(w: Workload, chunk: int = 16) -> dict:
    """Algorithmic FLOPs and compulsory HBM bytes of one prefill of ``w``.

    Per token and head: 6KV flops for the three state contractions (W.S, Q+.S and
    the rank-16 state update) plus 2C(3K+2V) for the in-chunk products (A, P, W,
    U and P.Delta). Compulsory bytes: q, k, v, out in the io dtype, g and beta in
    fp32 (g is K values per token and head, or one for a scalar gate), plus every
    initial and final state read or written (fp32).
    """
    K, V, C = w.head_k, w.head_v, chunk
    th = w.total_tokens * w.heads
    flops = th * (6 * K * V + 2 * C * (3 * K + 2 * V))
    es = 2 if w.bf16 else 4
    gate_bytes = 4 if w.gate == "scalar" else 4 * K
    bytes_tok = es * (2 * K + V) + gate_bytes + 4 + es * V
    states = w.num_seqs * w.heads * K * V * 4
    n_states = 1 + (1 if w.has_initial_state else 0)
    return {"flops": flops, "bytes": th * bytes_tok + n_states * states,
            "bytes_per_token_head": bytes_tok, "token_heads": th}
