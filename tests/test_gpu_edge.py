"""GPU parity at the recurrence's edge values, against the fp64 oracle.

The workloads' random inputs never reach the method's degenerate cases, so these
tests set them on purpose:

* beta = 0 with g = 0 (alpha = 1): every write vanishes, so the state never changes
  and o_t = S0^T q_t. The final state must equal the initial state bit for bit.
* beta = 1 with exactly unit-norm keys (bf16 values +-1/8 on 64 channels, or +-1/4 on
  16): the write replaces the state's component along k_t, so S_t^T k_t = v_t, and
  with q_t = k_t every output equals its value row (the backward keeps the
  workload's queries).
* g = 0: the plain delta rule, no decay.
* Strong decay, from per-token g = -8 (the in-chunk gates still fit the factored
  form) to -10, -30 and -1000 (per-pair form), a mix of channels, a chunk-local burst
  (both forms in one launch) and the scalar gate.

Each case runs the two-kernel prefill, the single-kernel form (bitwise equal to it)
and, where the sizes allow, the fp32 path, and the backward pass."""
import numpy as np
import pytest

from linear_attention_04_amd import inputs
from tests import gpu_util as gu
from tests import rounding_model

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_04_amd import kda

    kda.load_library()  # fails loudly when the HIP library is missing


def _case(name, seed, H=3, T=100, K=128, io="bf16", gate_kind="channel", lengths=None):
    w = inputs.custom_workload(name, seed, heads=H, total_tokens=T, head_k=K, head_v=K, io_dtype=io,
                               has_initial_state=True, lengths=lengths, gate=gate_kind)
    return w, inputs.generate(w)


def _unit_keys(shape, seed):
    """Keys of exactly unit norm in bf16 (and fp32): n channels of +-1/sqrt(n), with
    n = 64 (K >= 64) or 16, on a random support per token and head."""
    rng = np.random.default_rng([seed, 4242])
    T, H, K = shape
    n = 64 if K >= 64 else 16
    k = np.zeros(shape, np.float32)
    for t in range(T):
        for h in range(H):
            idx = rng.choice(K, size=n, replace=False)
            k[t, h, idx] = rng.choice(np.array([-1.0, 1.0], np.float32), size=n) / np.float32(np.sqrt(n))
    assert np.all(np.sum(k.astype(np.float64) ** 2, axis=-1) == 1.0)
    return k


def _edit(x, case, seed):
    """The inputs of edge case `case` (a fresh dict; x is not modified)."""
    x = dict(x)
    for key in ("q", "k", "v", "g", "beta"):
        x[key] = np.array(x[key], copy=True)
    g = x["g"]
    if case == "beta0_gate0":
        x["beta"][:] = 0.0
        g[:] = 0.0
    elif case == "beta1_unit_keys":
        x["k"] = _unit_keys(x["k"].shape, seed)
        x["q"] = x["k"].copy()
        x["beta"][:] = 1.0
    elif case == "beta1_unit_keys_q":
        # the same writes with the workload's queries: not parallel to the keys, so
        # the initial state still reaches the outputs and has a gradient
        x["k"] = _unit_keys(x["k"].shape, seed)
        x["beta"][:] = 1.0
    elif case == "beta1_unit_keys_gate0":
        x["k"] = _unit_keys(x["k"].shape, seed)
        x["q"] = x["k"].copy()
        x["beta"][:] = 1.0
        g[:] = 0.0
    elif case == "gate0":
        g[:] = 0.0
    elif case == "decay_mixed":
        # a tenth of the channels (or tokens, for a scalar gate) decay at -60 per token
        rng = np.random.default_rng([seed, 4243])
        g[rng.random(g.shape) < 0.1] = -60.0
    elif case == "decay_burst":
        # one channel of one chunk decays at -20 per token; every other chunk keeps
        # the workload's gates, so both gate forms run in one launch
        if g.ndim == 3:
            g[32:48, :, 5] = -20.0
        else:
            g[32:48, :] = -20.0
    elif case.startswith("decay"):
        g[:] = -float(case[len("decay"):])
    else:
        raise ValueError(case)
    return x


FORWARD_CASES = ["beta0_gate0", "beta1_unit_keys", "beta1_unit_keys_gate0", "gate0", "decay8", "decay10",
                 "decay30", "decay1000", "decay_mixed", "decay_burst"]


def _forward(w, x, packed=False, fused=True):
    torch = gu.torch_mod()
    d = gu.upload(x, w.bf16, packed)
    out, fs = gu.run_gpu(d)
    ro, rs = gu.run_oracle(x, packed)
    gu.assert_close("out", gu.to_host(out), ro, w.bf16)
    gu.assert_close("final_state", gu.to_host(fs), rs, w.bf16)
    if w.bf16:  # the rounding model takes the per-pair path where the kernels do
        mo, mfs = rounding_model.forward(x if packed else dict(x, cu_seqlens=None))
        gu.assert_model_band("out", gu.to_host(out), ro, mo)
        gu.assert_model_band("final_state", gu.to_host(fs), rs, mfs)
    if fused and w.bf16:
        from linear_attention_04_amd import kda

        out_f, fs_f = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                                        initial_state=d["initial_state"], fused=True)
        torch.cuda.synchronize()
        assert torch.equal(out_f, out) and torch.equal(fs_f, fs), "single-kernel form differs from the split"
    return d, out, fs


@pytest.mark.parametrize("case", FORWARD_CASES)
def test_edge_forward_bf16(case):
    w, x = _case(f"edge_{case}", 501, H=3, T=100)
    x = _edit(x, case, 501)
    print(f"case {case}: bf16 H=3 T=100", flush=True)
    torch = gu.torch_mod()
    d, out, fs = _forward(w, x)
    if case == "beta0_gate0":
        assert torch.equal(fs, d["initial_state"]), "beta = 0, g = 0 must leave the state unchanged"
    if case.startswith("beta1_unit_keys"):
        gu.assert_close("out vs v", gu.to_host(out), x["v"].astype(np.float64), True)


@pytest.mark.parametrize("case", ["beta0_gate0", "beta1_unit_keys", "decay30", "decay_burst"])
def test_edge_forward_bf16_packed(case):
    w, x = _case(f"edge_packed_{case}", 502, H=2, lengths=[40, 17, 0, 64, 5])
    x = _edit(x, case, 502)
    print(f"case {case}: bf16 packed", flush=True)
    _forward(w, x, packed=True)


@pytest.mark.parametrize("case", ["decay10", "decay1000", "decay_mixed", "decay_burst"])
def test_edge_forward_scalar_gate(case):
    w, x = _case(f"edge_sg_{case}", 503, H=3, T=90, gate_kind="scalar")
    x = _edit(x, case, 503)
    print(f"case {case}: bf16 scalar gate", flush=True)
    _forward(w, x)


@pytest.mark.parametrize("K", [16, 128])
@pytest.mark.parametrize("case", ["beta0_gate0", "beta1_unit_keys", "gate0", "decay10", "decay1000"])
def test_edge_forward_f32(K, case):
    w, x = _case(f"edge_f32_{case}", 504, H=2, T=53, K=K, io="f32")
    x = _edit(x, case, 504)
    print(f"case {case}: f32 K={K}", flush=True)
    torch = gu.torch_mod()
    d, out, fs = _forward(w, x, fused=False)
    if case == "beta0_gate0":
        assert torch.equal(fs, d["initial_state"]), "beta = 0, g = 0 must leave the state unchanged"


def _assert_grads(x, got, ref):
    """The backward's bars. dg is measured against the products it is summed from
    (gu.dg_term_scale): at these edge values it is many times smaller than they are.
    A gradient whose reference is zero (it reaches only through decays below fp64's
    range) must come out zero to within 1e-6."""
    scale = gu.dg_term_scale(x, ref)
    for name in GRADS:
        g, r = gu.to_host(got[name]), ref[name]
        if float(np.max(np.abs(r))) < 1e-30 and (name != "dg" or float(np.max(scale)) < 1e-30):
            m = float(np.max(np.abs(g)))
            print(f"  {name}: reference zero, max|got|={m:.3e}", flush=True)
            assert np.all(np.isfinite(g)) and m <= 1e-6, name
        elif name == "dg":
            gu.assert_dg_close(g, r, scale)
        else:
            gu.assert_close_rel(name, g, r)


# beta = 1 with q = k is left out here: every output then equals its value row
# whatever the initial state, so d_initial_state is zero by that identity up to
# rounding, and only the rounding noise would be compared
@pytest.mark.parametrize("case", ["beta0_gate0", "beta1_unit_keys_q", "gate0", "decay8", "decay10", "decay30",
                                  "decay1000", "decay_mixed", "decay_burst"])
def test_edge_backward(case):
    w, x = _case(f"edge_bwd_{case}", 505, H=3, T=100)
    x = _edit(x, case, 505)
    d_out, d_fs = inputs.output_gradients(w)
    print(f"case backward {case}: bf16 H=3 T=100", flush=True)
    d = gu.upload_backward(x, d_out, d_fs, False)
    got = gu.run_gpu_backward(d)
    ref = gu.run_oracle_backward(x, d_out, d_fs, False)
    _assert_grads(x, got, ref)


@pytest.mark.parametrize("case", ["decay30", "decay_burst"])
def test_edge_backward_scalar_gate(case):
    w, x = _case(f"edge_bwd_sg_{case}", 506, H=2, T=70, gate_kind="scalar")
    x = _edit(x, case, 506)
    d_out, d_fs = inputs.output_gradients(w)
    print(f"case backward {case}: bf16 scalar gate", flush=True)
    d = gu.upload_backward(x, d_out, d_fs, False)
    got = gu.run_gpu_backward(d)
    ref = gu.run_oracle_backward(x, d_out, d_fs, False)
    _assert_grads(x, got, ref)
