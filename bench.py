#!/usr/bin/env python3
"""Chunked KDA prefill benchmark on one MI355X.

One step is one whole prefill (intra-chunk kernel, then the recurrent inter-chunk
kernel) of the H=64, T=8192, K=V=128 bf16 workload with every input already in
device memory. Prints one JSON line with tokens/s, the dominant kernel's roofline
and the fp64 CPU oracle timed on the host cores as a baseline.

    python bench.py [--gpus 1] [--steps 200] [--warmup 100]

The default warm-up is long enough for the GPU clock to settle: from idle, the step
time takes about 40 back-to-back steps to reach its steady value.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "fixed_h64_t8192"
SCALAR_GATE_WORKLOAD = "fixed_h64_t8192_scalar_gate"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")

# Algorithmic bytes per (token, head) of each kernel at K = V = 128 (bf16 io):
#  intra: reads q, k (bf16) + g (fp32) + beta = 2*128 + 2*128 + 4*128 + 4 = 1028
#         (520 with a scalar gate: g is one fp32 per token and head),
#         writes its per-chunk record 14848 B / 16 tokens = 928;
#  inter: reads the record (928) and v (256), writes out (256), plus the fp32
#         final state (and initial state, if any) per (sequence, head).
INTRA_BYTES_PER_TH = {"channel": 1028 + 928, "scalar": 520 + 928}
INTER_BYTES_PER_TH = 928 + 256 + 256
STATE_BYTES = 128 * 128 * 4

# Backward kernels, algorithmic bytes per (token, head):
#  records:    q, k, g, beta in (1028; 520 scalar gate), forward + backward records
#              out ((14848 + 12800) / 16 = 1728);
#  states:     forward record (928) and v (256) in, every chunk's start state out
#              (bf16, 32768 B / 16 tokens = 2048), plus the initial state if any;
#  state_grad: backward record (800) and d_out (256) in, every chunk's end-state
#              gradient out (2048), plus d_final_state in and d_initial_state out;
#  token_grad: q, k, v, d_out (1024), g (512; 4 scalar), beta (4) and both stored
#              states (4096) in; dq, dk, dv (768), dg (512; 4 scalar), dbeta (4) out.
BWD_BYTES_PER_TH = {
    "records": {"channel": 1028 + 1728, "scalar": 520 + 1728},
    "states": {"channel": 928 + 256 + 2048, "scalar": 928 + 256 + 2048},
    "state_grad": {"channel": 800 + 256 + 2048, "scalar": 800 + 256 + 2048},
    "token_grad": {"channel": 1024 + 512 + 4 + 4096 + 768 + 512 + 4, "scalar": 1024 + 4 + 4 + 4096 + 768 + 4 + 4},
}


# Untimed steps before the warm-up: from idle the clocks take ~40 back-to-back steps
# (~20 ms) to settle, so a short warm-up alone would time the ramp. The timed region is
# still exactly the K steps after the W warm-up steps.
SETTLE_MS = 100.0


def settle(step) -> int:
    """Run untimed steps until SETTLE_MS of wall time has passed; returns how many."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return n


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="prefill workload (default: the H=64, T=8192 benchmark shape); see inputs.WORKLOADS")
    ap.add_argument("--gate", choices=("channel", "scalar"), default="channel",
                    help="scalar: the same shape with one gate per token and head (Gated DeltaNet)")
    ap.add_argument("--mode", choices=("prefill", "decode", "backward", "train"), default="prefill",
                    help="decode: one-token state update of --decode-batch sequences x 64 heads; "
                         "backward: the gradients of the prefill (kda_chunk_prefill_backward, four stages); "
                         "train: one training step, kda_chunk_prefill_for_backward then the reverse pass and the "
                         "token gradients on its workspace")
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--fused", action="store_true",
                    help="time the single-kernel form (kda_chunk_prefill_fused) instead of the split")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (to scale HBM counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch."""
    import torch

    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": {"read": 1 << 30, "write": 1 << 30},
                      "launches": 5}))
    return 0


def source_digest(tag: str) -> str:
    from linear_attention_04_amd import rocprof_report

    return rocprof_report.source_digest(rocprof_report.KERNEL_SOURCES[tag])


def profile_for(tag: str, workload: str):
    """The committed counter summary of kernel `tag` on `workload`
    (profiles/traffic_<tag>_<workload>.json, written by linear_attention_04_amd.rocprof_report),
    if it was taken on the kernel's current sources; else None."""
    path = os.path.join(PROFILES, f"traffic_{tag}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("source_digest") != source_digest(tag):
        return None
    return doc


def traffic_for(tag: str, workload: str):
    """Measured HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE), or None."""
    doc = profile_for(tag, workload)
    return None if doc is None else doc.get("hbm_bytes_per_launch")


def mfma_busy_for(tag: str, workload: str):
    """Share of SIMD cycles the matrix cores were busy in kernel `tag`
    (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE / 8), or None."""
    doc = profile_for(tag, workload)
    sq = None if doc is None else doc.get("sq_counters_per_dispatch")
    if not sq or not sq.get("GRBM_GUI_ACTIVE"):
        return None
    return sq.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * sq["GRBM_GUI_ACTIVE"] / 8)


def cpu_baseline(x, w, min_seconds: float = 10.0, max_repeats: int = 64):
    """The fp64 oracle as it stands, on the host cores. One pass over the whole
    workload takes well under a second on a many-core host, so the sample is the
    whole workload repeated until about `min_seconds` of CPU time have passed."""
    import oracle

    threads = oracle.max_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                       cu_seqlens=x["cu_seqlens"] if w.num_seqs > 1 else None,
                       initial_state=x["initial_state"], want_out=True, want_state=True)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or runs >= max_repeats:
            break
    return {
        "value": runs * w.total_tokens / dt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"whole workload ({w.heads} heads x {w.total_tokens} tokens) run {runs} times, {dt:.2f} s",
    }


def decode_bench(args):
    """One decode step (kda_decode_step) of B sequences x 64 heads per timed step;
    state [B, 64, 128, 128] fp32 read and written in place."""
    import numpy as np
    import torch

    from linear_attention_04_amd import inputs, kda

    B, H = args.decode_batch, 64
    w = inputs.custom_workload(f"decode_b{B}_h{H}", 1, H, B, gate=args.gate)
    x = inputs.generate(w)
    rng = np.random.default_rng([1, 7])
    s0 = (0.02 * rng.standard_normal((B, H, 128, 128))).astype(np.float32)
    dev = lambda a, bf: (torch.from_numpy(inputs.bf16_bits(a)).to("cuda").view(torch.bfloat16)  # noqa: E731
                         if bf else torch.from_numpy(a).to("cuda"))
    q, k, v = dev(x["q"], True), dev(x["k"], True), dev(x["v"], True)
    g, beta = dev(x["g"], False), dev(x["beta"], False)
    state = torch.from_numpy(s0).to("cuda")
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    dims = kda.KdaDims(B, H, 128, 128, B, kda.KDA_IO_BF16,
                       kda.KDA_GATE_SCALAR if args.gate == "scalar" else kda.KDA_GATE_CHANNEL)

    def step():
        st = kda.kda_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                 state.data_ptr(), out.data_ptr(), dims, stream.cuda_stream)
        if st:
            raise kda.KdaError(st, "decode")

    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    # Nothing runs between the warm-up and the timed steps but the synchronisation (the
    # checks and event allocations come first): an idle GPU lowers its clocks within
    # milliseconds, and the first timed steps would pay for it.
    settle_steps = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for i in range(args.steps):
        step()
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = float(np.mean([bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]))
    ms_step = wall * 1e3 / args.steps
    gate_bytes = 4 if args.gate == "scalar" else 512
    per_bh = 2 * 128 * 128 * 4 + 4 * 256 + gate_bytes + 4  # state in + out, q k v out, g, beta
    alg = per_bh * B * H
    achieved = alg / (kern_ms * 1e-3) / 1e9
    rec = {
        "metric": "KDA decode step tokens/s (one token per sequence, state update in place)",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_steps": settle_steps, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "head_k": 128, "head_v": 128, "gate": args.gate},
        "kernels_ms": {"decode": kern_ms},
        "roofline": {"kernel": "decode", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_for("decode", w.name), "algorithmic_bytes": alg,
                     "source_digest": source_digest("decode")},
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.max_threads()
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=np.arange(B + 1),
                           initial_state=s0)
            runs += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or runs >= 10000:
                break
        rec["cpu_baseline"] = {"value": runs * B / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"the whole step ({B} sequences x {H} heads) run {runs} times, {dt:.2f} s"}
    print(json.dumps(rec), flush=True)
    return 0


def backward_bench(args, w, x):
    """One step = one whole backward (its four stages) of workload ``w``."""
    import numpy as np
    import torch

    from linear_attention_04_amd import inputs, kda

    d_out_h, d_fs_h = inputs.output_gradients(w)
    dev = lambda a, bf: (torch.from_numpy(inputs.bf16_bits(a)).to("cuda").view(torch.bfloat16)  # noqa: E731
                         if bf else torch.from_numpy(a).to("cuda"))
    q, k, v = dev(x["q"], True), dev(x["k"], True), dev(x["v"], True)
    g, beta = dev(x["g"], False), dev(x["beta"], False)
    d_out, d_fs = dev(d_out_h, True), dev(d_fs_h, False)
    T, H, N = w.total_tokens, w.heads, w.num_seqs
    cu = torch.from_numpy(x["cu_seqlens"]).to("cuda") if N > 1 else None
    s0 = None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).to("cuda")
    cu_p = None if cu is None else cu.data_ptr()
    s0_p = None if s0 is None else s0.data_ptr()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
    ds0 = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    dims = kda.make_dims(q, v, cu, g=g)
    nbytes = kda.kda_backward_workspace_bytes(dims)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731

    # ev: the events recorded after each of the four stages; the step's start is the
    # previous step's last event
    def step(ev=None):
        rec = (lambda i: ev[i - 1].record(stream)) if ev is not None else (lambda i: None)
        st = [kda.kda_backward_records(P(q), P(k), P(g), P(beta), cu_p, dims, P(ws), nbytes, sp)]
        rec(1)
        st.append(kda.kda_backward_states(P(v), cu_p, s0_p, dims, P(ws), nbytes, sp))
        rec(2)
        st.append(kda.kda_backward_state_grad(P(d_out), cu_p, P(d_fs), P(ds0), dims, P(ws), nbytes, sp))
        rec(3)
        st.append(kda.kda_backward_token_grad(P(q), P(k), P(v), P(g), P(beta), P(d_out), cu_p, P(dq), P(dk),
                                              P(dv), P(dg), P(dbeta), dims, P(ws), nbytes, sp))
        rec(4)
        bad = [e for e in st if e]
        if bad:
            raise kda.KdaError(bad[0], "backward")

    step()
    torch.cuda.synchronize()
    if not all(bool(torch.isfinite(t.float()).all()) for t in (dq, dk, dv, dg, dbeta)):
        print("non-finite gradient", file=sys.stderr)
        return 1
    start = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    # Nothing runs between the warm-up and the timed steps but the synchronisation (the
    # checks and event allocations come first): an idle GPU lowers its clocks within
    # milliseconds, and the first timed steps would pay for it.
    settle_steps = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ("records", "states", "state_grad", "token_grad")
    marks = [[start if j == 0 else evs[j - 1][3]] + evs[j] for j in range(args.steps)]  # 5 per step
    stage_ms = {n: float(np.mean([m[i].elapsed_time(m[i + 1]) for m in marks])) for i, n in enumerate(names)}
    ms_step = wall * 1e3 / args.steps
    th = T * H
    n_s0 = 1 if s0 is not None else 0
    extra_states = {"records": 0, "states": n_s0, "state_grad": 2, "token_grad": 0}
    kern_bytes = {n: BWD_BYTES_PER_TH[n][w.gate] * th + extra_states[n] * STATE_BYTES * N * H for n in names}
    dom = max(names, key=lambda n: stage_ms[n])
    achieved = kern_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    digest = source_digest("bwd_" + dom)
    gate_bytes = 4 if w.gate == "scalar" else 512
    compulsory = th * (4 * 256 + gate_bytes + 4 + 3 * 256 + gate_bytes + 4) + (n_s0 + 2) * STATE_BYTES * N * H
    path_gbs = compulsory / (ms_step * 1e-3) / 1e9
    rec = {
        "metric": (f"KDA prefill backward tokens/s (gradients of q, k, v, g, beta, initial state), "
                   f"H={H} T={T} K=V=128 bf16" + (" (scalar gate)" if w.gate == "scalar" else "")),
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_steps": settle_steps, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "heads": H, "tokens": T, "head_k": 128, "head_v": 128, "num_seqs": N,
                   "initial_state": s0 is not None, "chunk": 16, "gate": w.gate, "pass": "backward"},
        "path_hbm": {"algorithmic_bytes": compulsory, "achieved": path_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": path_gbs / HBM_PEAK_GBS},
        "kernels_ms": stage_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for("bwd_" + dom, w.name),
                     "algorithmic_bytes": kern_bytes[dom], "source_digest": digest},
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.max_threads()
        heads = list(range(min(H, threads)))
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_out_h,
                            cu_seqlens=x["cu_seqlens"] if N > 1 else None, initial_state=x["initial_state"],
                            d_final_state=d_fs_h, heads=heads, threads=threads)
            runs += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or runs >= 64:
                break
        rec["cpu_baseline"] = {
            "value": runs * T * len(heads) / H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(heads)} of {H} heads x {T} tokens run {runs} times in {dt:.2f} s, "
                      f"scaled to all {H} heads"}
    print(json.dumps(rec), flush=True)
    return 0


def train_bench(args, w, x):
    """One step = one training step of workload ``w``: the forward that fills the
    backward workspace (kda_chunk_prefill_for_backward: records, then one recurrent
    pass for the output, final state and saved chunk states), then the reverse pass
    and the token gradients on that workspace."""
    import numpy as np
    import torch

    from linear_attention_04_amd import inputs, kda

    d_out_h, d_fs_h = inputs.output_gradients(w)
    dev = lambda a, bf: (torch.from_numpy(inputs.bf16_bits(a)).to("cuda").view(torch.bfloat16)  # noqa: E731
                         if bf else torch.from_numpy(a).to("cuda"))
    q, k, v = dev(x["q"], True), dev(x["k"], True), dev(x["v"], True)
    g, beta = dev(x["g"], False), dev(x["beta"], False)
    d_out, d_fs = dev(d_out_h, True), dev(d_fs_h, False)
    T, H, N = w.total_tokens, w.heads, w.num_seqs
    cu = torch.from_numpy(x["cu_seqlens"]).to("cuda") if N > 1 else None
    s0 = None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).to("cuda")
    cu_p = None if cu is None else cu.data_ptr()
    s0_p = None if s0 is None else s0.data_ptr()
    out = torch.empty_like(v)
    fs = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
    ds0 = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    dims = kda.make_dims(q, v, cu, g=g)
    nbytes = kda.kda_backward_workspace_bytes(dims)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731

    def step(ev=None):
        rec = (lambda i: ev[i - 1].record(stream)) if ev is not None else (lambda i: None)
        st = [kda.kda_chunk_prefill_for_backward(P(q), P(k), P(v), P(g), P(beta), cu_p, s0_p, P(out), P(fs), dims,
                                                 P(ws), nbytes, sp)]
        rec(1)
        st.append(kda.kda_backward_state_grad(P(d_out), cu_p, P(d_fs), P(ds0), dims, P(ws), nbytes, sp))
        rec(2)
        st.append(kda.kda_backward_token_grad(P(q), P(k), P(v), P(g), P(beta), P(d_out), cu_p, P(dq), P(dk),
                                              P(dv), P(dg), P(dbeta), dims, P(ws), nbytes, sp))
        rec(3)
        bad = [e for e in st if e]
        if bad:
            raise kda.KdaError(bad[0], "training step")

    step()
    torch.cuda.synchronize()
    if not all(bool(torch.isfinite(t.float()).all()) for t in (out, dq, dk, dv, dg, dbeta)):
        print("non-finite output or gradient", file=sys.stderr)
        return 1
    start = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    # Nothing runs between the warm-up and the timed steps but the synchronisation (the
    # checks and event allocations come first): an idle GPU lowers its clocks within
    # milliseconds, and the first timed steps would pay for it.
    settle_steps = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ("forward", "state_grad", "token_grad")
    marks = [[start if j == 0 else evs[j - 1][2]] + evs[j] for j in range(args.steps)]  # 4 per step
    stage_ms = {n: float(np.mean([m[i].elapsed_time(m[i + 1]) for m in marks])) for i, n in enumerate(names)}
    ms_step = wall * 1e3 / args.steps
    th = T * H
    n_s0 = 1 if s0 is not None else 0
    # the forward stage is two kernels: the records (as the backward's records stage)
    # and one recurrence that reads the forward record and v and writes out and every
    # chunk's start state
    kern_bytes = {"forward": (BWD_BYTES_PER_TH["records"][w.gate] + 928 + 256 + 2048 + 256) * th
                  + (2 * n_s0 + 1) * STATE_BYTES * N * H,
                  "state_grad": BWD_BYTES_PER_TH["state_grad"][w.gate] * th + 2 * STATE_BYTES * N * H,
                  "token_grad": BWD_BYTES_PER_TH["token_grad"][w.gate] * th}
    dom = max(names, key=lambda n: stage_ms[n])
    achieved = kern_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    traffic, digest = None, None
    if dom != "forward":  # one kernel, with its own counter summary
        digest = source_digest("bwd_" + dom)
        traffic = traffic_for("bwd_" + dom, w.name)
    gate_bytes = 4 if w.gate == "scalar" else 512
    forward_compulsory = th * (3 * 256 + gate_bytes + 4 + 256) + (2 * n_s0 + 1) * STATE_BYTES * N * H
    backward_compulsory = th * (4 * 256 + gate_bytes + 4 + 3 * 256 + gate_bytes + 4) + (n_s0 + 2) * STATE_BYTES * N * H
    compulsory = forward_compulsory + backward_compulsory
    path_gbs = compulsory / (ms_step * 1e-3) / 1e9
    rec = {
        "metric": (f"KDA training step tokens/s (prefill forward and its backward), H={H} T={T} K=V=128 bf16"
                   + (" (scalar gate)" if w.gate == "scalar" else "")),
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_steps": settle_steps, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "heads": H, "tokens": T, "head_k": 128, "head_v": 128, "num_seqs": N,
                   "initial_state": s0 is not None, "chunk": 16, "gate": w.gate, "pass": "train"},
        "path_hbm": {"algorithmic_bytes": compulsory, "achieved": path_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": path_gbs / HBM_PEAK_GBS},
        "kernels_ms": stage_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": kern_bytes[dom], "source_digest": digest},
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.max_threads()
        heads = list(range(min(H, threads)))
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=x["cu_seqlens"] if N > 1 else None,
                           initial_state=x["initial_state"], heads=heads, threads=threads)
            oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_out_h,
                            cu_seqlens=x["cu_seqlens"] if N > 1 else None, initial_state=x["initial_state"],
                            d_final_state=d_fs_h, heads=heads, threads=threads)
            runs += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or runs >= 64:
                break
        rec["cpu_baseline"] = {
            "value": runs * T * len(heads) / H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(heads)} of {H} heads x {T} tokens, forward and backward, run {runs} times in "
                      f"{dt:.2f} s, scaled to all {H} heads"}
    print(json.dumps(rec), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (heads and packed "
              "sequences would shard across GPUs without communication).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from linear_attention_04_amd import inputs, kda

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        return copy_calibration()
    kda.load_library()
    if args.mode == "decode":
        return decode_bench(args)
    if args.gate == "scalar":
        w = inputs.custom_workload(SCALAR_GATE_WORKLOAD, 1, 64, 8192, gate="scalar")
    else:
        w = inputs.WORKLOADS[args.workload]
    if not w.bf16:
        print("bench.py times the bf16 path; the fp32 workload is a parity case", file=sys.stderr)
        return 2
    x = inputs.generate(w)
    if args.mode == "backward":
        return backward_bench(args, w, x)
    if args.mode == "train":
        return train_bench(args, w, x)
    dev = lambda a, bf: (torch.from_numpy(inputs.bf16_bits(a)).to("cuda").view(torch.bfloat16)  # noqa: E731
                         if bf else torch.from_numpy(a).to("cuda"))
    q, k, v = dev(x["q"], True), dev(x["k"], True), dev(x["v"], True)
    g, beta = dev(x["g"], False), dev(x["beta"], False)
    T, H, N = w.total_tokens, w.heads, w.num_seqs
    cu = torch.from_numpy(x["cu_seqlens"]).to("cuda") if N > 1 else None
    s0 = None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).to("cuda")
    cu_p = None if cu is None else cu.data_ptr()
    s0_p = None if s0 is None else s0.data_ptr()
    n_states = 1 + (s0 is not None)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    dims = kda.make_dims(q, v, cu, g=g)
    ws = kda.workspace_for(dims, "cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    # Timed steps record an event between the two kernels (`mid`) and one at the end
    # (`end`); a step's end event is also the next step's start, so the kernels of
    # consecutive steps are separated by one event marker.
    def step(mid=None, end=None):
        if args.fused:
            st = kda.kda_chunk_prefill_fused(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                             cu_p, s0_p, out.data_ptr(), fs.data_ptr(), dims, ws.data_ptr(),
                                             ws.numel(), sp)
            if end is not None:
                end.record(stream)
            if st:
                raise kda.KdaError(st, "fused prefill")
            return
        st = kda.kda_intra_chunk(q.data_ptr(), k.data_ptr(), g.data_ptr(), beta.data_ptr(), cu_p, dims,
                                 ws.data_ptr(), ws.numel(), sp)
        if mid is not None:
            mid.record(stream)
        st2 = kda.kda_inter_chunk(v.data_ptr(), cu_p, s0_p, out.data_ptr(), fs.data_ptr(), dims, ws.data_ptr(),
                                  ws.numel(), sp)
        if end is not None:
            end.record(stream)
        if st or st2:
            raise kda.KdaError(st or st2, "prefill")

    step()
    torch.cuda.synchronize()
    if not bool(torch.isfinite(out.float()).all()):
        print("non-finite output", file=sys.stderr)
        return 1

    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    # Nothing runs between the warm-up and the timed steps but the synchronisation (the
    # checks and event allocations come first): an idle GPU lowers its clocks within
    # milliseconds, and the first timed steps would pay for it.
    settle_steps = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for i in range(args.steps):
        step(None if args.fused else mids[i], bounds[i + 1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.fused:
        intra_ms = float(np.mean([bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]))
        inter_ms = 0.0
    else:
        intra_ms = float(np.mean([bounds[i].elapsed_time(mids[i]) for i in range(args.steps)]))
        inter_ms = float(np.mean([mids[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]))
    ms_step = wall * 1e3 / args.steps

    counts = inputs.algorithmic_counts(w)
    th = T * H
    tokens_s = T / (ms_step * 1e-3)
    tflops = counts["flops"] / (ms_step * 1e-3) / 1e12
    path_gbs = counts["bytes"] / (ms_step * 1e-3) / 1e9

    # per kernel: mean launch time and its own algorithmic bytes (what it must read and
    # write, including the intermediate records)
    kernels = {
        "intra": (intra_ms, INTRA_BYTES_PER_TH[w.gate] * th),
        "inter": (inter_ms, INTER_BYTES_PER_TH * th + STATE_BYTES * w.num_seqs * H * n_states),
    }
    if args.fused:
        # one launch; its algorithmic bytes are the path's compulsory bytes
        kernels = {"fused": (intra_ms, counts["bytes"])}
    dom = max(kernels, key=lambda n: kernels[n][0])
    dom_ms, own_bytes = kernels[dom]
    # The roofline's algorithmic bytes are the method's compulsory bytes per token and
    # head (q, k, v, out bf16; g, beta fp32: 1540 at K = V = 128) times the token-heads
    # one launch processes, plus the states it must read or write, over the dominant
    # kernel's mean launch time; the kernel's own bytes (records included) are beside it.
    achieved = counts["bytes"] / (dom_ms * 1e-3) / 1e9
    own_achieved = own_bytes / (dom_ms * 1e-3) / 1e9
    digest = source_digest(dom)
    traffic = traffic_for(dom, w.name)
    mfma_busy = mfma_busy_for(dom, w.name)

    rec = {
        "metric": (f"KDA prefill tokens/s + TFLOP/s (% roofline), H={H} T={T} K=V=128 bf16"
                   + (" (scalar gate)" if w.gate == "scalar" else "") + (" (single-kernel ablation)" if args.fused else "")),
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": H, "tokens": T, "head_k": 128, "head_v": 128,
                   "num_seqs": N, "initial_state": s0 is not None, "chunk": 16, "gate": w.gate,
                   "kernels": "fused" if args.fused else "split"},
        "tflops": tflops,
        "tflops_frac": tflops / BF16_PEAK_TFLOPS,
        "path_hbm": {"algorithmic_bytes": counts["bytes"], "achieved": path_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": path_gbs / HBM_PEAK_GBS},
        "kernels_ms": {"fused": intra_ms} if args.fused else {"intra": intra_ms, "inter": inter_ms},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": counts["bytes"], "ms": dom_ms,
                     "kernel_own_bytes": own_bytes, "kernel_own_frac": own_achieved / HBM_PEAK_GBS,
                     "mfma_busy": mfma_busy, "source_digest": digest},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
