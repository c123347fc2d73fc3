"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times (one kda_chunk_prefill call over the whole batch). The 8192-token workloads
are compared element by element over every head; the 131072-token workload on a
sample of heads, which the oracle evaluates one by one."""
import numpy as np
import pytest

import oracle
from linear_attention_04_amd import inputs
from tests import gpu_util as gu
from tests import rounding_model

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()


def _run(name, keep, w=None, model=False):
    """model: also hold the GPU's error to the bf16 rounding model's on the same heads."""
    w = w or inputs.WORKLOADS[name]
    print(f"workload {name}: heads kept for the oracle {keep}", flush=True)
    dev, host = gu.generate_on_device(w, keep)
    out, fs = gu.run_gpu(dev)
    packed = w.num_seqs > 1
    ro, rs = oracle.prefill(host["q"], host["k"], host["v"], host["g"], host["beta"],
                            cu_seqlens=host["cu_seqlens"] if packed else None,
                            initial_state=host["initial_state"])
    got_o = gu.to_host(out[:, keep])
    got_s = gu.to_host(fs[:, keep])
    gu.assert_close("out", got_o, ro, True)
    gu.assert_close("final_state", got_s, rs, True)
    if model:
        mo, mfs = rounding_model.forward(host if packed else dict(host, cu_seqlens=None))
        gu.assert_model_band("out", got_o, ro, mo)
        gu.assert_model_band("final_state", got_s, rs, mfs)


@pytest.mark.parametrize("name", ["fixed_h64_t8192", "fixed_h96_t8192_s0", "varlen_h96_t8192_n8"])
def test_fullsize_all_heads(name):
    # the headline workload is also held to the rounding model (~30 s of CPU)
    _run(name, list(range(inputs.WORKLOADS[name].heads)), model=name == "fixed_h64_t8192")


def test_fullsize_long_context_sampled_heads():
    """Eight of the 64 heads, one on each XCD (the recurrent kernel places (sequence,
    head) pair p on XCD p mod 8) and spread over the head range; every head runs the
    same 2-tile workgroup form, so the sample covers each distinct launch position."""
    _run("long_h64_t131072_s0", [0, 9, 18, 27, 36, 45, 54, 63])


def test_fullsize_scalar_gate_all_heads():
    """The scalar-gated delta rule at the benchmark shape (g [T, H])."""
    w = inputs.custom_workload("fixed_h64_t8192_scalar_gate", 1, 64, 8192, gate="scalar")
    _run(w.name, list(range(64)), w)


def test_fused_fullsize_equals_split():
    """The single-kernel ablation at the benchmark shape, bitwise against the split."""
    import torch

    from linear_attention_04_amd import kda

    w = inputs.WORKLOADS["fixed_h64_t8192"]
    dev, _ = gu.generate_on_device(w, [])
    out_s, fs_s = gu.run_gpu(dev)
    out_f, fs_f = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], fused=True)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_f) and torch.equal(fs_s, fs_f)


@pytest.mark.parametrize("name", ["fixed_h64_t8192", "fixed_h96_t8192_s0", "varlen_h96_t8192_n8"])
def test_training_forward_fullsize_equals_prefill(name):
    """kda_chunk_prefill_for_backward over a whole workload gives kda_chunk_prefill's
    output and final state bit for bit. Its recurrence stages the saved chunk states
    (2-tile form, 64 pairs) or the outputs (4-tile form, beyond 64 pairs) in LDS for a
    store wave, here over 512 chunks per sequence."""
    import torch

    from linear_attention_04_amd import kda

    w = inputs.WORKLOADS[name]
    print(f"workload {name}", flush=True)
    dev, _ = gu.generate_on_device(w, [])
    out_p, fs_p = gu.run_gpu(dev)
    out_t, fs_t, ws = kda.chunk_prefill_for_backward(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                                     cu_seqlens=dev["cu_seqlens"],
                                                     initial_state=dev["initial_state"])
    torch.cuda.synchronize()
    del ws
    assert torch.equal(out_p, out_t) and torch.equal(fs_p, fs_t)


def _backward_fullsize(name, keep, w=None):
    """The backward at a full workload: one kda_chunk_prefill_backward call over the
    whole batch (as the benchmark times it); the oracle's gradients for the heads in
    ``keep``, and over every head the identities <dq, q> = <dO, o> and
    <dv, v> + <dS0, S0> = <dO, o> + <dS_T, S_T> against this library's own forward."""
    w = w or inputs.WORKLOADS[name]
    print(f"backward {name}: heads kept for the oracle {keep}", flush=True)
    dev, host = gu.generate_on_device(w, keep)
    d_out_h, d_fs_h = inputs.output_gradients(w)
    dev["d_out"] = gu.to_device(d_out_h, True)
    dev["d_final_state"] = gu.to_device(d_fs_h, False)
    got = gu.run_gpu_backward(dev)
    packed = w.num_seqs > 1
    ref = oracle.backward(host["q"], host["k"], host["v"], host["g"], host["beta"],
                          np.ascontiguousarray(d_out_h[:, keep]),
                          cu_seqlens=host["cu_seqlens"] if packed else None, initial_state=host["initial_state"],
                          d_final_state=np.ascontiguousarray(d_fs_h[:, keep]))
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        gu.assert_close_rel(n, gu.to_host(got[n][:, keep]), ref[n])
    gu.assert_close_rel("d_initial_state", gu.to_host(got["d_initial_state"][:, keep]), ref["d_initial_state"])
    out, fs = gu.run_gpu(dev)
    f64 = lambda t: t.double()  # noqa: E731
    l_out = float((f64(out) * f64(dev["d_out"])).sum())
    l_all = l_out + float((fs.double() * dev["d_final_state"].double()).sum())
    lhs_q = float((f64(got["dq"]) * f64(dev["q"])).sum())
    lhs_v = float((f64(got["dv"]) * f64(dev["v"])).sum())
    if dev["initial_state"] is not None:
        lhs_v += float((got["d_initial_state"].double() * dev["initial_state"].double()).sum())
    print(f"  <dq,q>={lhs_q:.6e} <dO,o>={l_out:.6e}  <dv,v>+<dS0,S0>={lhs_v:.6e} L={l_all:.6e}", flush=True)
    assert abs(lhs_q - l_out) <= 1e-2 * abs(l_out)
    assert abs(lhs_v - l_all) <= 1e-2 * abs(l_all)


def test_backward_fullsize_sampled_heads():
    _backward_fullsize("fixed_h64_t8192", [0, 21, 42, 63])


def test_backward_fullsize_varlen_with_state():
    _backward_fullsize("varlen_h96_t8192_n8", [5, 50, 95])


def test_backward_fullsize_h96_with_state():
    _backward_fullsize("fixed_h96_t8192_s0", [0, 47, 95])


def test_backward_fullsize_long_context_sampled_heads():
    """131 072 tokens of 64 heads (about 60 GB of device memory with the workspace's
    chunk states); the oracle evaluates two heads."""
    _backward_fullsize("long_h64_t131072_s0", [7, 56])
