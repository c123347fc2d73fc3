"""The bf16 rounding model (tests/rounding_model.py): its algebra pinned to the fp64
oracle, and its error predictions for the prefill workloads and the backward pass.

The GPU parity tests hold the HIP path to the model's prediction on their own inputs
(gpu_util.assert_model_band); the predictions pinned here set the backward tolerances
in gpu_util (BWD_REL_L2, BWD_MAX_REL)."""
import numpy as np
import pytest

import oracle
from linear_attention_04_amd import inputs
from tests import gpu_util as gu
from tests import rounding_model as rm


def _oracle_fwd(x):
    return oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=x["cu_seqlens"],
                          initial_state=x["initial_state"])


def _oracle_bwd(x, d_out, d_fs):
    return oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_out, cu_seqlens=x["cu_seqlens"],
                           initial_state=x["initial_state"], d_final_state=d_fs)


def _max_rel(got, ref):
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def test_bf16_rounding():
    # round to nearest, ties to even, on exact bf16 neighbours of 1
    e = 2.0 ** -8
    vals = np.array([1.0, 1 + e, 1 + 3 * e, 1 + 1.5 * e, -(1 + e), 1 + e - 2.0 ** -20])
    want = np.array([1.0, 1.0, 1 + 4 * e, 1 + 2 * e, -1.0, 1.0])
    assert np.array_equal(rm.bf16(vals), want)
    # and the shared input generator's rounding on random values
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32) * 3
    assert np.array_equal(rm.bf16(x), inputs.round_to_bf16(x).astype(np.float64))


@pytest.mark.parametrize("case", ["packed_state", "scalar_gate", "strong_decay"])
def test_exact_model_is_the_oracle(case):
    """With every rounding off the model is the chunked algebra, equal to the token
    loop: forward and backward, ragged chunks, empty sequences, the per-pair path."""
    if case == "packed_state":
        w = inputs.custom_workload("m_packed", 201, heads=2, head_k=128, head_v=128, has_initial_state=True,
                                   lengths=[1, 15, 16, 0, 37, 64])
    elif case == "scalar_gate":
        w = inputs.custom_workload("m_scalar", 202, heads=2, total_tokens=90, gate="scalar")
    else:
        w = inputs.custom_workload("m_decay", 203, heads=2, total_tokens=70, gate_scale=8.0,
                                   has_initial_state=True)
    x = inputs.generate(w)
    o, fs = _oracle_fwd(x)
    mo, mfs = rm.forward(x, exact=True)
    assert np.max(np.abs(mo - o)) <= 1e-10 * max(1.0, np.max(np.abs(o)))
    assert np.max(np.abs(mfs - fs)) <= 1e-10 * max(1.0, np.max(np.abs(fs)))
    d_out, d_fs = inputs.output_gradients(w)
    ref = _oracle_bwd(x, d_out, d_fs)
    got = rm.backward(x, d_out, d_fs, exact=True)
    for name, r in ref.items():
        assert np.max(np.abs(got[name] - r)) <= 1e-9 * max(1.0, np.max(np.abs(r))), name


def test_strong_decay_takes_the_pair_path():
    """A chunk whose running gate strays more than the factored span from its 8th
    token is formed pair by pair (the factored form would overflow to inf * 0)."""
    w = inputs.custom_workload("m_decay2", 204, heads=1, total_tokens=32, gate_scale=30.0)
    x = inputs.generate(w)
    mo, mfs = rm.forward(x)
    assert np.all(np.isfinite(mo)) and np.all(np.isfinite(mfs))
    o, fs = _oracle_fwd(x)
    assert rm.rel_l2(mo, o) < 5e-3


# Reduced forms of the prefill workloads: the same value recipes, fewer heads and
# tokens (the error statistics do not depend on the head count, and are stationary
# after the gates' memory, a few chunks).
FORWARD_CASES = {
    "fixed_h64_t8192": (dict(total_tokens=2048), (2.0e-3, 2.7e-3), (1.2e-3, 1.9e-3)),
    "fixed_h96_t8192_s0": (dict(total_tokens=2048, has_initial_state=True), (2.0e-3, 2.7e-3), (1.2e-3, 1.9e-3)),
    "varlen_h96_t8192_n8": (dict(total_tokens=2048, num_seqs=8), (2.0e-3, 2.7e-3), (1.2e-3, 1.9e-3)),
    "long_h64_t131072_s0": (dict(total_tokens=4096, gate_scale=0.02, has_initial_state=True), (2.6e-3, 3.5e-3),
                            (1.4e-3, 2.1e-3)),
}


@pytest.mark.parametrize("name", list(FORWARD_CASES))
def test_forward_error_prediction(name):
    """Predicted rel-L2 of out and of the final state against the oracle: inside the
    bands below, and below the 5e-3 bar with room to spare."""
    kw, out_band, state_band = FORWARD_CASES[name]
    w = inputs.custom_workload("pred_" + name, 300 + len(name), heads=4, **kw)
    x = inputs.generate(w)
    o, fs = _oracle_fwd(x)
    mo, mfs = rm.forward(x)
    e_out, e_state = rm.rel_l2(mo, o), rm.rel_l2(mfs, fs)
    print(f"{name}: out rel-L2 {e_out:.3e} max {np.max(np.abs(mo - o)):.3e}; state rel-L2 {e_state:.3e}")
    assert out_band[0] <= e_out <= out_band[1]
    assert state_band[0] <= e_state <= state_band[1]
    assert e_out <= 0.75 * gu.BF16_REL_L2 and np.max(np.abs(mo - o)) <= 0.1 * gu.BF16_MAX_ABS


def test_design_choices_are_what_the_error_rests_on():
    """Coarser plans the model rejects: one bf16 term for A and P (no split), and the
    state update's Delta as one bf16 term. Each raises the predicted error."""
    w = inputs.custom_workload("pred_plans", 310, heads=4, total_tokens=1024)
    x = inputs.generate(w)
    o, _ = _oracle_fwd(x)
    base = rm.rel_l2(rm.forward(x)[0], o)

    class OneTermAP(rm._Round):
        def hl_product(self, a, b):
            return rm.bf16(a) @ rm._t(rm.bf16(b))

    class OneTermDelta(rm._Round):
        def two(self, x):
            return rm.bf16(x)

    for plan in (OneTermAP, OneTermDelta):
        worse = rm.rel_l2(rm.forward(x, rounding=plan(False))[0], o)
        print(f"{plan.__name__}: {worse:.3e} against {base:.3e}")
        assert worse > 1.15 * base


BACKWARD_CASES = {
    "fixed": dict(total_tokens=1024),
    "long_memory": dict(total_tokens=2048, gate_scale=0.02, has_initial_state=True),
}


@pytest.mark.parametrize("name", list(BACKWARD_CASES))
def test_backward_error_prediction(name):
    """Predicted errors of every gradient: rel-L2 1.5e-3 .. 3.8e-3 and max|err| below
    4.5e-3 of the tensor's largest magnitude. The backward bars in gpu_util keep 30%
    (rel-L2) and 2x (max|err|, which grows with the tensor size) over the largest."""
    w = inputs.custom_workload("predb_" + name, 320 + len(name), heads=4, **BACKWARD_CASES[name])
    x = inputs.generate(w)
    d_out, d_fs = inputs.output_gradients(w)
    ref = _oracle_bwd(x, d_out, d_fs)
    got = rm.backward(x, d_out, d_fs)
    for key, r in ref.items():
        rel, mx = rm.rel_l2(got[key], r), _max_rel(got[key], r)
        print(f"{name} {key}: rel-L2 {rel:.3e} max|err|/max|ref| {mx:.3e}")
        assert 1.5e-3 <= rel <= 3.8e-3, key
        assert mx <= 4.5e-3, key
        assert rel <= gu.BWD_REL_L2 / 1.3 and mx <= gu.BWD_MAX_REL / 2, key
