"""kda.chunk_kda, the autograd entry: its forward equals kda_chunk_prefill and its
gradients equal kda_chunk_prefill_backward bit for bit (both run the HIP kernels;
the backward ones are checked against the oracle in test_gpu_backward.py), for
L = <d_out, out> + <d_final_state, final_state> formed by torch ops on its outputs."""
import pytest

from linear_attention_04_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GRADS = ("q", "k", "v", "g", "beta")


@pytest.fixture(scope="module")
def kda_mod():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()  # fails loudly when the HIP library is missing
    return kda


def _leaves(d, names):
    return {n: (d[n].clone().requires_grad_(True) if d[n] is not None else None) for n in names}


@pytest.mark.parametrize("case", ["packed_with_state", "scalar_gate_no_state"])
def test_gradients_equal_the_backward_entry(kda_mod, case):
    torch = gu.torch_mod()
    if case == "packed_with_state":
        w = inputs.custom_workload("ag_packed", 701, heads=3, lengths=[40, 0, 77, 1], has_initial_state=True)
    else:
        w = inputs.custom_workload("ag_scalar", 702, heads=2, total_tokens=90, gate="scalar")
    packed = w.num_seqs > 1
    print(f"case {case}: H={w.heads} T={w.total_tokens} N={w.num_seqs}", flush=True)
    x = inputs.generate(w)
    d_out, d_fs = inputs.output_gradients(w)
    d = gu.upload_backward(x, d_out, d_fs, packed)
    leaf = _leaves(d, GRADS + ("initial_state",))
    out, fs = kda_mod.chunk_kda(leaf["q"], leaf["k"], leaf["v"], leaf["g"], leaf["beta"],
                                cu_seqlens=d["cu_seqlens"], initial_state=leaf["initial_state"])
    loss = (out.float() * d["d_out"].float()).sum() + (fs * d["d_final_state"]).sum()
    loss.backward()
    torch.cuda.synchronize()

    ref_out, ref_fs = gu.run_gpu(d)
    assert torch.equal(out.detach(), ref_out) and torch.equal(fs.detach(), ref_fs)
    ref = gu.run_gpu_backward(d)
    for n in GRADS:
        assert leaf[n].grad is not None and leaf[n].grad.dtype == d[n].dtype, n
        assert torch.equal(leaf[n].grad, ref["d" + n]), n
    if leaf["initial_state"] is not None:
        assert torch.equal(leaf["initial_state"].grad, ref["d_initial_state"])


def test_output_only_loss(kda_mod):
    """Only out enters the loss (final state not returned): the final state's gradient
    is zero, as kda_chunk_prefill_backward with no d_final_state."""
    torch = gu.torch_mod()
    w = inputs.custom_workload("ag_out_only", 703, heads=2, total_tokens=53, has_initial_state=True)
    x = inputs.generate(w)
    d_out, _ = inputs.output_gradients(w)
    d = gu.upload_backward(x, d_out, None, False)
    leaf = _leaves(d, GRADS)  # the initial state needs no gradient here
    out, fs = kda_mod.chunk_kda(leaf["q"], leaf["k"], leaf["v"], leaf["g"], leaf["beta"],
                                initial_state=d["initial_state"], output_final_state=False)
    assert fs is None
    (out.float() * d["d_out"].float()).sum().backward()
    torch.cuda.synchronize()
    ref = gu.run_gpu_backward(d, want_d_initial_state=False)
    for n in GRADS:
        assert torch.equal(leaf[n].grad, ref["d" + n]), n


def test_without_gradients_it_is_the_prefill(kda_mod):
    torch = gu.torch_mod()
    w = inputs.custom_workload("ag_nograd", 704, heads=2, total_tokens=70, has_initial_state=True)
    x = inputs.generate(w)
    d = gu.upload(x, True, False)
    ref_out, ref_fs = gu.run_gpu(d)
    out, fs = kda_mod.chunk_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"])
    assert not out.requires_grad
    leaf = _leaves(d, ("q",))
    with torch.no_grad():
        out2, fs2 = kda_mod.chunk_kda(leaf["q"], d["k"], d["v"], d["g"], d["beta"],
                                      initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert not out2.requires_grad
    for o, f in ((out, fs), (out2, fs2)):
        assert torch.equal(o, ref_out) and torch.equal(f, ref_fs)
