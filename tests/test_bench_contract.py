"""bench.py's output contract: the one-GPU refusal, the CPU baseline object (on the
CPU, with a tiny workload) and, on a GPU, one JSON line per mode with every field a
reader of the benchmark relies on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")

TOP_KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "scaling", "vs_baseline", "dtype", "data", "config", "roofline"}
ROOFLINE_KEYS = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_object():
    sys.path.insert(0, ROOT)
    import bench
    from linear_attention_04_amd import inputs

    w = inputs.custom_workload("tiny_baseline", 3, heads=2, total_tokens=40)
    x = inputs.generate(w)
    cb = bench.cpu_baseline(x, w, min_seconds=0.05, max_repeats=3)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1 and isinstance(cb["sample"], str)


def test_source_digest_ignores_comments():
    """A profile's traffic figures stay valid across comment edits of its kernel sources
    (the compiled code is the same), and not across a change of code."""
    sys.path.insert(0, ROOT)
    from linear_attention_04_amd.rocprof_report import code_text

    base = 'int a = 1;\nchar *s = "x // y /* z */";\nchar q = \'"\';\nint b;'
    edited = ('// header\nint a = 1;  // one\n\n/* a block\n   comment */\nchar *s = "x // y /* z */";\n'
              'char q = \'"\';   \nint b; /* end */\n')
    assert code_text(edited).replace(" ", "") == code_text(base).replace(" ", "")
    assert code_text(base) == base
    assert code_text(base.replace("1", "2")) != code_text(base)
    assert code_text('char *s = "a /* b";  // c */ d') == 'char *s = "a /* b";'


def _run_bench(*args):
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "2", "--no-cpu-baseline", *args],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
@pytest.mark.parametrize("args", [(), ("--gate", "scalar"), ("--mode", "decode"), ("--mode", "backward"),
                                  ("--mode", "train")],
                         ids=["prefill", "scalar_gate", "decode", "backward", "train"])
def test_bench_json_line(args):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = _run_bench(*args)
    assert TOP_KEYS <= set(d), TOP_KEYS - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    r = d["roofline"]
    assert ROOFLINE_KEYS <= set(r), ROOFLINE_KEYS - set(r)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert "cpu_baseline" not in d
