"""rocprofv3 harness: kernel times, measured HBM traffic and matrix-core use of the
library's kernels under bench.py, against the MI355X peaks.

Two steps, both from the repository root:

    python -m linear_attention_04_amd.rocprof_report run [--only h64 ...] [--dir rocprof_out]
    python -m linear_attention_04_amd.rocprof_report summarize [--only h64 ...] [--dir rocprof_out]

``run`` (on the GPU machine) starts, for every profiled bench mode, four rocprofv3
passes over ``python3 bench.py`` as child processes: a kernel trace with statistics,
one counter pass for FETCH_SIZE, one for WRITE_SIZE and one for the SQ counters
(instruction mix and MFMA busy cycles). The counter passes use short runs. No pass
combines counters with tracing, and no pass asks for more counters than one
hardware pass collects. ``summarize`` turns the CSV files into ``profiles/<mode>.md``
(per kernel: calls, average / min / max duration, HBM bytes read and written, MFMA
busy and VALU+MFMA issue share of SIMD cycles) and into
``profiles/traffic_<tag>_<workload>.json``. bench.py quotes the latter as measured
traffic while its recorded source digest matches the kernel sources (their code;
comments do not count).

HBM bytes are the counters scaled by what they read for a plain device copy of known
size (``run --only copy``): FETCH_SIZE counts half the bytes a 128-byte request
moves, so reads scale by ~2.0; WRITE_SIZE scales by 1.0.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(PKG, "csrc")

# MI355X: 256 compute units of 4 SIMDs, dealt over 8 XCDs; GRBM_GUI_ACTIVE is summed
# over the XCDs, so one XCD's active cycles are GRBM_GUI_ACTIVE / 8.
SIMDS = 1024
XCDS = 8
HBM_PEAK_GBS = 8000.0

# Sources each kernel tag is built from: a traffic file is valid while their digest
# matches.
KERNEL_SOURCES = {
    "intra": ["kda_intra_bf16.hip", "kda_intra_wave.h", "kda_gate_exact.h", "kda_device.h", "kda_chunks.h"],
    "inter": ["kda_inter_bf16.hip", "kda_chain.h", "kda_ring.h", "kda_device.h", "kda_chunks.h"],
    "fused": ["kda_inter_bf16.hip", "kda_chain.h", "kda_ring.h", "kda_intra_wave.h", "kda_gate_exact.h",
              "kda_device.h", "kda_chunks.h"],
    "decode": ["kda_decode.hip", "kda_device.h"],
    "bwd_records": ["kda_intra_bf16.hip", "kda_intra_wave.h", "kda_gate_exact.h", "kda_device.h", "kda_chunks.h"],
    "bwd_states": ["kda_inter_bf16.hip", "kda_chain.h", "kda_ring.h", "kda_device.h", "kda_chunks.h"],
    "bwd_state_grad": ["kda_state_grad_bf16.hip", "kda_ring.h", "kda_device.h", "kda_chunks.h"],
    "bwd_token_grad": ["kda_grad_bf16.hip", "kda_gate_exact.h", "kda_ring.h", "kda_device.h", "kda_chunks.h"],
}

SQ_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU",
               "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"]


class Mode:
    """One profiled bench.py invocation."""

    def __init__(self, name, title, bench_args, workload, kernels, trace_steps=200, trace_warmup=100):
        self.name = name
        self.title = title
        self.bench_args = bench_args
        self.workload = workload
        self.kernels = kernels  # kernel base name -> (tag or None, label)
        self.trace_steps = trace_steps
        self.trace_warmup = trace_warmup


PREFILL = "KDA prefill, K=V=128 bf16"
MODES = {m.name: m for m in (
    Mode("h64", f"{PREFILL}, H=64 T=8192 (the headline workload)", ["--workload", "fixed_h64_t8192"],
         "fixed_h64_t8192", {"kda_intra_bf16_kernel": ("intra", ""), "kda_inter_bf16_kernel": ("inter", "")}),
    Mode("h96s0", f"{PREFILL}, H=96 T=8192, initial state", ["--workload", "fixed_h96_t8192_s0"],
         "fixed_h96_t8192_s0", {"kda_intra_bf16_kernel": ("intra", ""), "kda_inter_bf16_kernel": ("inter", "")}),
    Mode("varlen", f"{PREFILL}, H=96, 8 packed sequences of 8192 tokens", ["--workload", "varlen_h96_t8192_n8"],
         "varlen_h96_t8192_n8", {"kda_chunk_table_kernel": (None, ""), "kda_intra_bf16_kernel": ("intra", ""),
                                 "kda_inter_bf16_kernel": ("inter", "")}),
    Mode("long", f"{PREFILL}, H=64 T=131072, initial state", ["--workload", "long_h64_t131072_s0"],
         "long_h64_t131072_s0", {"kda_intra_bf16_kernel": ("intra", ""), "kda_inter_bf16_kernel": ("inter", "")},
         20, 20),
    Mode("sg", f"{PREFILL}, H=64 T=8192, scalar gate", ["--gate", "scalar"], "fixed_h64_t8192_scalar_gate",
         {"kda_intra_bf16_kernel": ("intra", ""), "kda_inter_bf16_kernel": ("inter", "")}),
    Mode("fused", f"{PREFILL}, H=64 T=8192, single-kernel ablation", ["--fused"], "fixed_h64_t8192",
         {"kda_fused_bf16_kernel": ("fused", "")}, 10, 10),
    Mode("decode", "KDA decode step, 64 sequences x 64 heads, K=V=128 bf16", ["--mode", "decode"], "decode_b64_h64",
         {"kda_decode_kernel": ("decode", "")}),
    Mode("bwd", "KDA prefill backward, H=64 T=8192 K=V=128 bf16", ["--mode", "backward"], "fixed_h64_t8192",
         {"kda_intra_bf16_kernel": ("bwd_records", " (records)"), "kda_inter_bf16_kernel": ("bwd_states", " (states)"),
          "kda_state_grad_bf16_kernel": ("bwd_state_grad", " (state_grad)"),
          "kda_grad_bf16_kernel": ("bwd_token_grad", " (token_grad)")}, 50, 50),
    Mode("train", "KDA training step (prefill forward and backward), H=64 T=8192 K=V=128 bf16", ["--mode", "train"],
         "fixed_h64_t8192",
         {"kda_intra_bf16_kernel": (None, " (records, in the forward)"),
          "kda_inter_bf16_kernel": (None, " (output and saved states, in the forward)"),
          "kda_state_grad_bf16_kernel": (None, " (state_grad)"), "kda_grad_bf16_kernel": (None, " (token_grad)")},
         50, 50),
)}
PROFILE_FILES = {
    "h64": "prefill_fixed_h64_t8192.md", "h96s0": "prefill_fixed_h96_t8192_s0.md",
    "varlen": "prefill_varlen_h96_t8192_n8.md", "long": "prefill_long_h64_t131072_s0.md",
    "sg": "prefill_scalar_gate_fixed_h64_t8192.md", "fused": "fused_prefill_fixed_h64_t8192.md",
    "decode": "decode_b64_h64.md", "bwd": "backward_fixed_h64_t8192.md", "train": "train_fixed_h64_t8192.md",
}


def code_text(src: str) -> str:
    """C++/HIP source without its comments, trailing blanks and empty lines: what the
    compiler sees. String and character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        ch = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif ch in "\"'":
            j = i + 1
            while j < n and src[j] != ch:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(ch)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def source_digest(names) -> str:
    """Digest of the code (not the comments) of the named kernel sources."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_base(raw: str):
    """'kda_..._kernel' from a demangled or mangled kernel name (the profiler leaves
    names with bf16 template arguments mangled, where digits run into the name)."""
    m = re.search(r"(kda_[a-z0-9_]+?_kernel)", raw)
    return m.group(1) if m else None


# ---------------------------------------------------------------------------
# passes

def commands(mode: Mode, out_dir: str):
    """(pass name, argv) of the four rocprofv3 passes of one mode."""
    bench = ["python3", "bench.py", *mode.bench_args, "--no-cpu-baseline"]
    d = lambda p: os.path.join(out_dir, f"{mode.name}_{p}")  # noqa: E731
    short = ["--steps", "2", "--warmup", "1"]
    # each pass under its own time limit (timeout signals rocprofv3 and the program it
    # runs); a counter pass that asked for too much would hang, so those are killed
    trace_limit = ["timeout", "-k", "10", "300"]
    pmc_limit = ["timeout", "-s", "KILL", "120"]
    return [
        ("trace", [*trace_limit, "rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", d("trace"),
                   "-o", "run", "--", *bench, "--steps", str(mode.trace_steps), "--warmup", str(mode.trace_warmup)]),
        ("fetch", [*pmc_limit, "rocprofv3", "--pmc", "FETCH_SIZE", "--output-format", "csv", "-d", d("fetch"), "-o",
                   "run", "--", *bench, *short]),
        ("write", [*pmc_limit, "rocprofv3", "--pmc", "WRITE_SIZE", "--output-format", "csv", "-d", d("write"), "-o",
                   "run", "--", *bench, *short]),
        ("sq", [*pmc_limit, "rocprofv3", "--pmc", *SQ_COUNTERS, "--output-format", "csv", "-d", d("sq"), "-o", "run",
                "--", *bench, *short]),
    ]


COPY_COMMANDS = [
    ("fetch", ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", "FETCH_SIZE", "--output-format", "csv", "-d",
               "{dir}/copy_fetch", "-o", "run", "--", "python3", "bench.py", "--copy-calibration"]),
    ("write", ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", "WRITE_SIZE", "--output-format", "csv", "-d",
               "{dir}/copy_write", "-o", "run", "--", "python3", "bench.py", "--copy-calibration"]),
]


def run(names, out_dir: str) -> int:
    """Every pass of every named mode as a child process, each under its own time
    limit; stops at the first failure (a failed or timed-out GPU step ends the run)."""
    os.makedirs(out_dir, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name in names:
        if name == "copy":
            cmds = [(p, [a.format(dir=out_dir) for a in argv]) for p, argv in COPY_COMMANDS]
        else:
            cmds = commands(MODES[name], out_dir)
        for pass_name, argv in cmds:
            print(f"== {name} {pass_name}: {' '.join(argv)}", flush=True)
            log = os.path.join(out_dir, f"{name}_{pass_name}.log")
            with open(log, "w") as f:
                r = subprocess.run(argv, cwd=ROOT, env=env, stdout=f, stderr=subprocess.STDOUT)
            if r.returncode in (124, 137):
                print(f"   timed out (see {log})", flush=True)
                return r.returncode
            # rocprofv3 may end with a fault of its own after the program has finished
            # and its results are whole: the CSV files decide
            ok = os.path.isdir(os.path.join(out_dir, f"{name}_{pass_name}"))
            print(f"   rc={r.returncode} results={'yes' if ok else 'no'}", flush=True)
            if not ok:
                return r.returncode or 1
    return 0


# ---------------------------------------------------------------------------
# summaries

def _csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def kernel_stats(d):
    out = {}
    for r in _csv(_find(d, "kernel_stats.csv")):
        k = kernel_base(r["Name"])
        if k is None:
            continue
        s = out.setdefault(k, {"calls": 0, "total_ns": 0.0, "min_ns": float("inf"), "max_ns": 0.0})
        calls = int(r["Calls"])
        s["calls"] += calls
        s["total_ns"] += float(r["AverageNs"]) * calls
        s["min_ns"] = min(s["min_ns"], float(r["MinNs"]))
        s["max_ns"] = max(s["max_ns"], float(r["MaxNs"]))
    for s in out.values():
        s["avg_us"] = s["total_ns"] / s["calls"] / 1e3
        s["min_us"] = s["min_ns"] / 1e3
        s["max_us"] = s["max_ns"] / 1e3
    return out


def counter_means(d):
    """{kernel: {counter: mean value per dispatch}}."""
    acc = {}
    for r in _csv(_find(d, "counter_collection.csv")):
        k = kernel_base(r["Kernel_Name"])
        if k is None:
            continue
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
        # a counter can be reported per XCD or instance: sum within the dispatch
        acc[k][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: {c: statistics.mean(v.values()) for c, v in cs.items()} for k, cs in acc.items()}


def calibration(in_dir):
    """(read scale, write scale) from the copy passes, or the factors measured on
    MI355X (2.0, 1.0) when they were not run."""
    try:
        f = copy_kernel_counter(os.path.join(in_dir, "copy_fetch"))
        w = copy_kernel_counter(os.path.join(in_dir, "copy_write"))
    except FileNotFoundError:
        f = w = None
    if not f or not w:
        return 1.9999498856704274, 1.0, "the factors of hbm_counter_calibration.md"
    moved_kib = float(1 << 20)  # 1 GiB each way per launch
    return moved_kib / f, moved_kib / w, "the copy passes of this run"


def copy_kernel_counter(d):
    """Mean counter value per dispatch of the device copy kernel in pass directory d."""
    per = {}
    for r in _csv(_find(d, "counter_collection.csv")):
        if "copy" in r["Kernel_Name"].lower():
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return statistics.mean(per.values()) if per else None


def bench_line(path):
    with open(path) as f:
        for line in f:
            if line.startswith('{"metric"'):
                return json.loads(line)
    return None


def summarize(names, in_dir: str, read_scale: float, write_scale: float, scale_src: str):
    for name in names:
        mode = MODES[name]
        d = lambda p: os.path.join(in_dir, f"{name}_{p}")  # noqa: E731
        st = kernel_stats(d("trace"))
        fe, wr = counter_means(d("fetch")), counter_means(d("write"))
        try:
            sq = counter_means(d("sq"))
        except FileNotFoundError:
            sq = {}
        b = bench_line(os.path.join(in_dir, f"{name}_trace.log")) or {}
        cmds = commands(mode, in_dir)
        lines = [f"# {mode.title}", "", f"Workload `{mode.workload}`. Made by "
                 "`python -m linear_attention_04_amd.rocprof_report run --only " + name + f" --dir {in_dir}` "
                 "(then `summarize`), which runs:", "", "```"]
        lines += [" ".join(argv) for _, argv in cmds]
        lines += ["```", "",
                  "| kernel | calls | avg us | min us | max us | HBM read MB | HBM write MB | MFMA busy | "
                  "VALU+MFMA issue |", "|---|---|---|---|---|---|---|---|---|"]
        for k, (tag, label) in mode.kernels.items():
            if k not in st:
                continue
            s = st[k]
            rd = fe.get(k, {}).get("FETCH_SIZE", 0.0) * 1024 * read_scale
            wb = wr.get(k, {}).get("WRITE_SIZE", 0.0) * 1024 * write_scale
            busy = issue = "-"
            q = sq.get(k)
            if q and q.get("GRBM_GUI_ACTIVE"):
                simd_cycles = SIMDS * q["GRBM_GUI_ACTIVE"] / XCDS
                mf = q.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
                valu = q.get("SQ_INSTS_VALU", 0.0) - q.get("SQ_INSTS_MFMA", 0.0)
                busy = f"{100 * mf / simd_cycles:.1f}%"
                issue = f"{100 * (4 * valu + mf) / simd_cycles:.1f}%"
            lines.append(f"| {k}{label} | {s['calls']} | {s['avg_us']:.1f} | {s['min_us']:.1f} | {s['max_us']:.1f} | "
                         f"{rd / 1e6:.1f} | {wb / 1e6:.1f} | {busy} | {issue} |")
            if tag:
                doc = {"kernel": tag, "workload": mode.workload, "sources": KERNEL_SOURCES[tag],
                       "source_digest": source_digest(KERNEL_SOURCES[tag]),
                       "fetch_size_kib_per_dispatch": fe.get(k, {}).get("FETCH_SIZE"),
                       "write_size_kib_per_dispatch": wr.get(k, {}).get("WRITE_SIZE"),
                       "read_scale": read_scale, "write_scale": write_scale,
                       "read_bytes_per_launch": rd, "write_bytes_per_launch": wb, "hbm_bytes_per_launch": rd + wb,
                       "avg_us": s["avg_us"]}
                if q:
                    doc["sq_counters_per_dispatch"] = q
                with open(os.path.join(PROFILES, f"traffic_{tag}_{mode.workload}.json"), "w") as f:
                    json.dump(doc, f, indent=1)
                    f.write("\n")
        lines += ["", f"HBM bytes: FETCH_SIZE x {read_scale:.4f} and WRITE_SIZE x {write_scale:.4f} "
                  f"({scale_src}). MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles "
                  f"({SIMDS} SIMDs x GRBM_GUI_ACTIVE / {XCDS}); VALU+MFMA issue: 4 cycles per non-MFMA VALU "
                  "instruction plus the MFMA busy cycles, over the same SIMD cycles (an estimate of how full the "
                  "SIMDs' issue is)."]
        if b:
            km = b.get("kernels_ms")
            lines += [f"bench.py's own HIP-event averages in the traced run (ms): {json.dumps(km)}; whole step "
                      f"{b['ms_per_step'] * 1e3:.1f} us, {b['value'] / 1e6:.2f} M tokens/s."]
        lines.append("")
        out = os.path.join(PROFILES, PROFILE_FILES[name])
        with open(out, "w") as f:
            f.write("\n".join(lines))
        print(out, {k: round(st[k]["avg_us"], 1) for k in mode.kernels if k in st})


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("step", choices=("run", "summarize"))
    ap.add_argument("--only", nargs="*", default=None, help=f"modes (default: all): {' '.join(MODES)} copy")
    ap.add_argument("--dir", default="rocprof_out", help="where the passes write (run) and are read from")
    a = ap.parse_args(argv)
    names = a.only or list(MODES)
    if a.step == "run":
        return run(names, a.dir)
    rs, ws, src = calibration(a.dir)
    summarize([n for n in names if n != "copy"], a.dir, rs, ws, src)
    return 0


if __name__ == "__main__":
    sys.exit(main())
