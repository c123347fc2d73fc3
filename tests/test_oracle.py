"""CPU pins of the fp64 oracle (no GPU)."""
import numpy as np
import pytest

import oracle
from linear_attention_04_amd import inputs
from oracle import reference
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle.prefill)


@pytest.mark.parametrize("check", oracle_pins.BACKWARD_CHECKS, ids=lambda f: f.__name__)
def test_backward_pin(check):
    check(oracle.backward)


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(10)
    lens = [5, 17, 1, 33, 16]
    T, H, K, V = sum(lens), 3, 8, 5
    q = rng.standard_normal((T, H, K)).astype(np.float32)
    k = (rng.standard_normal((T, H, K)) / np.sqrt(K)).astype(np.float32)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    g = (-0.2 * rng.random((T, H, K))).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    s0 = rng.standard_normal((len(lens), H, K, V)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, fs = oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=s0)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, fn = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], initial_state=s0[n:n + 1])
        assert np.array_equal(on, o[a:b])
        assert np.array_equal(fn[0], fs[n])


def test_split_and_resume_equals_one_run():
    rng = np.random.default_rng(11)
    T, H, K, V = 40, 2, 6, 7
    q = rng.standard_normal((T, H, K)).astype(np.float32)
    k = (rng.standard_normal((T, H, K)) / np.sqrt(K)).astype(np.float32)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    g = (-0.2 * rng.random((T, H, K))).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    o, fs = oracle.prefill(q, k, v, g, beta)
    for cut in (1, 13, 16, 39):
        o1, f1 = oracle.prefill(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut])
        o2, f2 = oracle.prefill(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:],
                                initial_state=f1.astype(np.float32))
        # the carried state is rounded to fp32 at the cut, as a caller would pass it
        assert np.max(np.abs(np.concatenate([o1, o2]) - o)) < 1e-5
        assert np.max(np.abs(f2 - fs)) < 1e-5
        assert np.array_equal(o1, o[:cut])


def test_head_subset_matches_full_run():
    w = inputs.custom_workload("t", 77, heads=5, total_tokens=50, head_k=8, head_v=4,
                               io_dtype="f32", has_initial_state=True, num_seqs=2)
    x = inputs.generate(w)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"])
    o, fs = oracle.prefill(*args, cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"])
    so, sfs = oracle.prefill(*args, cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                             heads=[4, 1])
    assert np.array_equal(so, o[:, [4, 1]])
    assert np.array_equal(sfs, fs[:, [4, 1]])


def test_chunked_intermediates_are_consistent():
    """The chunked form's pieces obey their defining identities: T is the inverse of
    I + A, A is strictly lower and P lower triangular, and Delta = U - W S0."""
    rng = np.random.default_rng(12)
    T, K, V = 40, 16, 16
    q = rng.standard_normal((T, K))
    k = rng.standard_normal((T, K)) / 4
    v = rng.standard_normal((T, V))
    g = -0.1 * rng.random((T, K))
    beta = rng.random(T)
    _, _, inter = reference.chunked(q, k, v, g, beta, rng.standard_normal((K, V)), intermediates=True)
    for it in inter:
        n = it["A"].shape[0]
        assert np.allclose(np.triu(it["A"]), 0)
        assert np.allclose(np.triu(it["P"], 1), 0)
        assert np.allclose(it["T"] @ (np.eye(n) + it["A"]), np.eye(n), atol=1e-12)
        assert np.allclose(it["Delta"], it["U"] - it["W"] @ it["S0"], atol=1e-12)


def test_bad_arguments_rejected():
    q = np.zeros((4, 1, 2), np.float32)
    v = np.zeros((4, 1, 3), np.float32)
    b = np.zeros((4, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.prefill(q, q, v, q, b, cu_seqlens=[0, 3, 2, 4])
    with pytest.raises(ValueError):
        oracle.prefill(q, q, v, q, b, cu_seqlens=[0, 5])
    with pytest.raises(ValueError):
        oracle.prefill(q, q, v, q, b, heads=[1])


def test_generator_is_deterministic_and_shaped():
    w = inputs.WORKLOADS["varlen_h96_t8192_n8"]
    lens = inputs.seq_lengths(w)
    assert lens.sum() == 8192 and len(lens) == 8
    assert np.all(lens >= 64) and np.all(lens % 16 != 0)
    small = inputs.custom_workload("s", 3, heads=2, total_tokens=100, has_initial_state=True)
    a, b = inputs.generate(small), inputs.generate(small)
    for key in ("q", "k", "v", "g", "beta", "initial_state"):
        assert np.array_equal(a[key], b[key])
    assert np.allclose(np.linalg.norm(a["k"], axis=-1), 1.0, atol=1e-2)
    assert np.allclose(np.linalg.norm(a["q"], axis=-1), 1.0 / np.sqrt(128), atol=1e-3)
    assert np.all(inputs.round_to_bf16(a["q"]) == a["q"])
    assert np.all(a["g"] <= 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e-39], np.float32)
    r = inputs.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                 # tie -> even
    assert r[2] == 1.0 + 4 * 2**-8     # tie -> even (up)
    assert r[3] == 1.0
    assert r[4] == -2.5


def test_oracle_matches_stored_golden():
    """Drift guard: the oracle still reproduces tests/golden/oracle_small_varlen.json."""
    import json
    import os

    from tests.golden import make_golden

    path = os.path.join(os.path.dirname(make_golden.__file__), "oracle_small_varlen.json")
    doc = json.load(open(path))
    x, o, fs = make_golden.compute()
    assert x["cu_seqlens"].tolist() == doc["cu_seqlens"]
    assert np.max(np.abs(o - np.array(doc["out"]))) <= 1e-14
    assert np.max(np.abs(fs - np.array(doc["final_state"]))) <= 1e-14


def test_scalar_gate_is_the_scalar_decay_delta_rule():
    """A [T, H] gate: the oracle must apply the token's one decay to every key channel,
    i.e. S <- (I - beta k k^T) (alpha S) + beta k v^T with a scalar alpha = exp(g),
    written out here with explicit K x K matrices for tiny sizes."""
    rng = np.random.default_rng(7)
    T, H, K, V = 9, 2, 4, 3
    q = rng.standard_normal((T, H, K)).astype(np.float32)
    k = rng.standard_normal((T, H, K)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    g = (-0.3 * rng.random((T, H))).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    s0 = rng.standard_normal((1, H, K, V)).astype(np.float32)
    out, fs = oracle.prefill(q, k, v, g, beta, initial_state=s0)
    for h in range(H):
        S = s0[0, h].astype(np.float64)
        for t in range(T):
            a = np.exp(np.float64(g[t, h]))
            kt = k[t, h].astype(np.float64)
            keep = np.eye(K) - np.float64(beta[t, h]) * np.outer(kt, kt)
            S = keep @ (a * S) + np.float64(beta[t, h]) * np.outer(kt, v[t, h].astype(np.float64))
            np.testing.assert_allclose(out[t, h], S.T @ q[t, h].astype(np.float64), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(fs[0, h], S, rtol=1e-12, atol=1e-13)


def test_scalar_gate_generator_shapes():
    w = inputs.custom_workload("sg", 5, 3, 40, head_k=16, head_v=16, io_dtype="f32", gate="scalar")
    x = inputs.generate(w)
    assert x["g"].shape == (40, 3) and np.all(x["g"] <= 0)
    w2 = inputs.custom_workload("cg", 5, 3, 40, head_k=16, head_v=16, io_dtype="f32")
    x2 = inputs.generate(w2)
    # the gate is drawn last in each block, so the other tensors are unchanged
    for name in ("q", "k", "v", "beta"):
        np.testing.assert_array_equal(x[name], x2[name])


def test_one_token_sequences_are_single_decode_steps():
    """A batch of one-token sequences from given states (the decode step's reading):
    each state takes exactly one step S <- (I - b k k^T) Diag(exp g) S + b k v^T and the
    output is S^T q, written out with explicit matrices."""
    rng = np.random.default_rng(17)
    B, H, K, V = 5, 2, 6, 4
    q = rng.standard_normal((B, H, K)).astype(np.float32)
    k = rng.standard_normal((B, H, K)).astype(np.float32)
    v = rng.standard_normal((B, H, V)).astype(np.float32)
    g = (-0.5 * rng.random((B, H, K))).astype(np.float32)
    beta = rng.random((B, H)).astype(np.float32)
    s0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    out, fs = oracle.prefill(q, k, v, g, beta, cu_seqlens=np.arange(B + 1), initial_state=s0)
    f = lambda a: np.asarray(a, np.float64)  # noqa: E731
    for b in range(B):
        for h in range(H):
            kk = f(k[b, h])
            S = (np.eye(K) - f(beta[b, h]) * np.outer(kk, kk)) @ np.diag(np.exp(f(g[b, h]))) @ f(s0[b, h]) \
                + f(beta[b, h]) * np.outer(kk, f(v[b, h]))
            np.testing.assert_allclose(fs[b, h], S, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(out[b, h], S.T @ f(q[b, h]), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("chunk,ref", [(1, 0), (4, 3), (16, 0), (16, 8), (16, 15), (64, 32)])
def test_chunked_backward_equals_oracle(chunk, ref):
    """The chunk-level backward algebra (the form the GPU kernels use) equals the
    token-by-token reverse pass, with a partial last chunk."""
    rng = np.random.default_rng(30 + chunk + ref)
    T, K, V = 45, 8, 6
    q = rng.standard_normal((T, 1, K)).astype(np.float32)
    k = (rng.standard_normal((T, 1, K)) / np.sqrt(K)).astype(np.float32)
    v = rng.standard_normal((T, 1, V)).astype(np.float32)
    g = (-0.3 * rng.random((T, 1, K))).astype(np.float32)
    beta = rng.random((T, 1)).astype(np.float32)
    do = rng.standard_normal((T, 1, V)).astype(np.float32)
    s0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    dsT = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    want = oracle.backward(q, k, v, g, beta, do, initial_state=s0, d_final_state=dsT)
    got = reference.chunked_backward(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], do[:, 0],
                                     s0[0, 0], dsT[0, 0], chunk=chunk, ref=ref)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.max(np.abs(got[name] - want[name][:, 0])) <= 1e-12, name
    assert np.max(np.abs(got["dS0"] - want["d_initial_state"][0, 0])) <= 1e-12


def test_backward_varlen_and_head_subset():
    """Packed sequences equal separate runs; a head subset equals the full run's rows."""
    rng = np.random.default_rng(31)
    lens = [5, 17, 0, 33]
    T, H, K, V = sum(lens), 3, 6, 5
    q = rng.standard_normal((T, H, K)).astype(np.float32)
    k = (rng.standard_normal((T, H, K)) / np.sqrt(K)).astype(np.float32)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    g = (-0.2 * rng.random((T, H, K))).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    do = rng.standard_normal((T, H, V)).astype(np.float32)
    s0 = rng.standard_normal((len(lens), H, K, V)).astype(np.float32)
    dsT = rng.standard_normal((len(lens), H, K, V)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    full = oracle.backward(q, k, v, g, beta, do, cu_seqlens=cu, initial_state=s0, d_final_state=dsT)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        one = oracle.backward(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], do[a:b],
                              initial_state=s0[n:n + 1], d_final_state=dsT[n:n + 1])
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.array_equal(one[name], full[name][a:b])
        assert np.array_equal(one["d_initial_state"][0], full["d_initial_state"][n])
    sub = oracle.backward(q, k, v, g, beta, do, cu_seqlens=cu, initial_state=s0, d_final_state=dsT,
                          heads=[2, 0])
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.array_equal(sub[name], full[name][:, [2, 0]])
