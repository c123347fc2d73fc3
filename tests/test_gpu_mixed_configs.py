"""GPU parity on a fixed, seeded sweep of mixed configurations: the features the other
tests take one at a time, drawn together. Head counts on both sides of the 2-tile /
4-tile switch of the recurrent kernels (more than 64 (sequence, head) pairs), packed
batches with empty and one-token sequences, both gate kinds, with and without initial
states; the forward for every case, the backward for those with K = V = 128 bf16."""
import numpy as np
import pytest

from linear_attention_04_amd import inputs
from tests import gpu_util as gu
from tests import rounding_model

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def _configs(n=16, seed=2026):
    """Gate scale cycles through 0.02 (long memory), 0.1 (the workloads') and 0.5 (|G_C|
    up to ~6 per chunk); every fourth case runs the fp32 path (K = V = 32)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        f32 = i % 4 == 3
        H = int(rng.choice([1, 2, 5, 17] if f32 else [1, 2, 5, 17, 33, 65, 70]))
        N = int(rng.integers(1, 7))
        lengths = [int(x) for x in rng.integers(0, 91, size=N)]
        if N > 2:
            lengths[int(rng.integers(0, N))] = 0
            lengths[int(rng.integers(0, N))] = 1
        if sum(lengths) == 0:
            lengths[0] = 23
        out.append(dict(i=i, H=H, lengths=lengths, gate=str(rng.choice(["channel", "scalar"])),
                        state=bool(rng.integers(0, 2)), scale=[0.02, 0.1, 0.5][i % 3],
                        io="f32" if f32 else "bf16"))
    return out


CONFIGS = _configs()


def _ids(c):
    return f"{c['i']}_h{c['H']}_n{len(c['lengths'])}_{c['gate']}_{'s0' if c['state'] else 'nos0'}_{c['io']}"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()  # fails loudly when the HIP library is missing


def _workload(c):
    K = 128 if c["io"] == "bf16" else 32
    return inputs.custom_workload(f"mixed_{c['i']}", 4000 + c["i"], heads=c["H"], head_k=K, head_v=K,
                                  io_dtype=c["io"], gate_scale=c["scale"], has_initial_state=c["state"],
                                  lengths=c["lengths"], gate=c["gate"])


@pytest.mark.parametrize("c", CONFIGS, ids=_ids)
def test_forward(c):
    w = _workload(c)
    print(f"case {_ids(c)}: lengths={c['lengths']} pairs={c['H'] * len(c['lengths'])}", flush=True)
    x = inputs.generate(w)
    d = gu.upload(x, w.bf16, True)
    out, fs = gu.run_gpu(d)
    ro, rs = gu.run_oracle(x, True)
    gu.assert_close("out", gu.to_host(out), ro, w.bf16)
    gu.assert_close("final_state", gu.to_host(fs), rs, w.bf16)
    if w.bf16:
        mo, mfs = rounding_model.forward(x)
        gu.assert_model_band("out", gu.to_host(out), ro, mo)
        gu.assert_model_band("final_state", gu.to_host(fs), rs, mfs)


@pytest.mark.parametrize("c", [c for c in CONFIGS if c["io"] == "bf16"], ids=_ids)
def test_backward(c):
    w = _workload(c)
    print(f"case {_ids(c)}: lengths={c['lengths']} pairs={c['H'] * len(c['lengths'])}", flush=True)
    x = inputs.generate(w)
    d_out, d_fs = inputs.output_gradients(w)
    d = gu.upload_backward(x, d_out, d_fs, True)
    got = gu.run_gpu_backward(d)
    ref = gu.run_oracle_backward(x, d_out, d_fs, True)
    model = rounding_model.backward(x, d_out, d_fs)
    for name in GRADS:
        gu.assert_close_rel(name, gu.to_host(got[name]), ref[name])
        gu.assert_model_band(name, gu.to_host(got[name]), ref[name], model[name])
