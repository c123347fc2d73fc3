"""GPU parity of the one-token decode step (kda_decode_step) against the fp64
oracle: a decode step is the recurrence over a single token per sequence, so the
oracle runs the batch as B packed one-token sequences from the given states."""
import numpy as np
import pytest

import oracle
from linear_attention_04_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# The step is fp32 arithmetic on an fp32 state, so the state is held to fp32-level
# accuracy (relative to its norm); bf16 outputs to the bf16 tolerance.
STATE_REL_L2 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()


def _batch(seed, B, H, io="bf16", gate="channel", state_scale=0.5):
    w = inputs.custom_workload(f"decode_b{B}_h{H}", seed, heads=H, total_tokens=B, io_dtype=io, gate=gate)
    x = inputs.generate(w)
    rng = np.random.default_rng([seed, 7])
    x["state"] = (state_scale * rng.standard_normal((B, H, 128, 128))).astype(np.float32)
    return w, x


def _oracle(x, B):
    return oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=np.arange(B + 1),
                          initial_state=x["state"])


def _gpu(x, bf16):
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    d = gu.upload(x, bf16, False)
    st = torch.from_numpy(x["state"]).to("cuda")
    out = kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st)
    torch.cuda.synchronize()
    return gu.to_host(out), gu.to_host(st)


def _check_state(got, ref):
    max_abs, rel = gu.errors(got, ref)
    print(f"  state: max|err|={max_abs:.3e} relL2={rel:.3e}", flush=True)
    assert rel <= STATE_REL_L2


@pytest.mark.parametrize("io,gate", [("bf16", "channel"), ("bf16", "scalar"), ("f32", "channel"), ("f32", "scalar")])
def test_decode_step(io, gate):
    B, H = 7, 5
    print(f"case decode io={io} gate={gate} B={B} H={H}", flush=True)
    w, x = _batch(11, B, H, io, gate)
    out, st = _gpu(x, w.bf16)
    ro, rs = _oracle(x, B)
    gu.assert_close("out", out, ro, w.bf16)
    _check_state(st, rs)


def test_decode_many_steps_equals_prefill_oracle():
    """40 consecutive decode steps of 3 sequences equal the oracle over the 40 tokens."""
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    B, H, T = 3, 4, 40
    print(f"case decode x{T} B={B} H={H}", flush=True)
    w = inputs.custom_workload("decode_seq", 21, heads=H, total_tokens=B * T, gate_scale=0.1)
    x = inputs.generate(w)
    # token t of sequence b is row b * T + t of the packed batch
    rng = np.random.default_rng(5)
    s0 = (0.1 * rng.standard_normal((B, H, 128, 128))).astype(np.float32)
    cu = np.arange(0, B * T + 1, T)
    ro, rs = oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=cu, initial_state=s0)
    d = gu.upload(x, True, False)
    st = torch.from_numpy(s0).to("cuda")
    outs = []
    for t in range(T):
        rows = torch.arange(B, device="cuda") * T + t
        pick = lambda a: a[rows].contiguous()  # noqa: E731
        outs.append(kda.decode_step(pick(d["q"]), pick(d["k"]), pick(d["v"]), pick(d["g"]), pick(d["beta"]), st))
    torch.cuda.synchronize()
    got = np.stack([gu.to_host(o) for o in outs], axis=1).reshape(B * T, H, 128)
    gu.assert_close("out", got, ro, True)
    _check_state(gu.to_host(st), rs)


def test_decode_continues_a_prefill():
    """Prefill 100 tokens on the GPU, then decode token 101 from the final state."""
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    H, T = 4, 101
    w = inputs.custom_workload("prefill_then_decode", 23, heads=H, total_tokens=T)
    x = inputs.generate(w)
    ro, rs = oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"])
    d = gu.upload(x, True, False)
    head = {n: d[n][:T - 1].contiguous() for n in ("q", "k", "v", "g", "beta")}
    _, fs = kda.chunk_prefill(head["q"], head["k"], head["v"], head["g"], head["beta"])
    tail = {n: d[n][T - 1:].contiguous() for n in ("q", "k", "v", "g", "beta")}
    out = kda.decode_step(tail["q"], tail["k"], tail["v"], tail["g"], tail["beta"], fs)
    torch.cuda.synchronize()
    gu.assert_close("out", gu.to_host(out), ro[T - 1:], True)
    gu.assert_close("final_state", gu.to_host(fs), rs, True)


def test_decode_full_batch():
    """The benchmark shape: 64 sequences x 64 heads."""
    B, H = 64, 64
    print(f"case decode B={B} H={H}", flush=True)
    w, x = _batch(31, B, H)
    out, st = _gpu(x, True)
    ro, rs = _oracle(x, B)
    gu.assert_close("out", out, ro, True)
    _check_state(st, rs)


def test_decode_empty_batch():
    from linear_attention_04_amd import kda

    d = kda.KdaDims(0, 4, 128, 128, 0, kda.KDA_IO_BF16, kda.KDA_GATE_CHANNEL)
    assert kda.kda_decode_step(None, None, None, None, None, None, None, d, None) == kda.KDA_OK


def test_decode_graph_replay():
    """The decode step captured in a HIP graph: each replay advances the state in place
    and equals an eager step from the same state."""
    from linear_attention_04_amd import kda

    torch = gu.torch_mod()
    B, H = 5, 4
    w, x = _batch(41, B, H)
    d = gu.upload(x, True, False)
    st = torch.from_numpy(x["state"]).to("cuda")
    out = torch.empty_like(d["v"])
    kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st.clone(), out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st, out=out)
    for rep in range(3):
        ref_state = st.clone()
        ref_out = kda.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], ref_state)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(st, ref_state), f"replay {rep} differs"
