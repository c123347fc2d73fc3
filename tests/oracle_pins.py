"""Checks that pin the fp64 oracle to facts other than itself.

Each check takes an oracle entry point (same signature as ``oracle.prefill``) so
the same battery can be run against deliberately broken copies of the oracle
(tests/test_oracle_mutations.py) to show that a plausible slip fails at least
one of them. Each check raises AssertionError on failure.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import reference


def _rand_case(rng, T, K, V, with_state=True, gate=0.3):
    q = rng.standard_normal((T, 1, K)).astype(np.float32)
    k = rng.standard_normal((T, 1, K)).astype(np.float32) / np.float32(math.sqrt(K))
    v = rng.standard_normal((T, 1, V)).astype(np.float32)
    g = (-gate * rng.random((T, 1, K))).astype(np.float32)
    beta = rng.random((T, 1)).astype(np.float32)
    s0 = (rng.standard_normal((1, 1, K, V)) * 0.5).astype(np.float32) if with_state else None
    return q, k, v, g, beta, s0


def check_hand_example(run):
    """K=2, V=3, three tokens, worked by hand (decay of 1/2 enters as the fp32
    value of ln(1/2), so values after a decay carry a relative 2e-9 offset).

    t=1: k=(1,0) v=(2,3,4) g=(0,0) beta=1 q=(1,1): S'=S0=[[1,0,2],[0,1,0]], pred=(1,0,2),
         delta=(1,3,2), S=[[2,3,4],[0,1,0]], o=(2,4,4).
    t=2: k=(0,1) v=(1,1,1) g=(ln1/2,0) beta=1/2 q=(1,2): S'=[[1,1.5,2],[0,1,0]], pred=(0,1,0),
         delta=(0.5,0,0.5), S=[[1,1.5,2],[0.5,1,0.5]], o=(2,3.5,3).
    t=3: k=(1/2,1/2) v=(0,2,-2) g=(0,ln1/2) beta=1 q=(1,-1): S'=[[1,1.5,2],[0.25,0.5,0.25]],
         pred=(0.625,1,1.125), delta=(-0.625,1,-3.125),
         S=[[0.6875,2,0.4375],[-0.0625,1,-1.3125]], o=(0.75,1,1.75).
    """
    half = math.log(0.5)
    q = np.array([[1, 1], [1, 2], [1, -1]], np.float32)[:, None, :]
    k = np.array([[1, 0], [0, 1], [0.5, 0.5]], np.float32)[:, None, :]
    v = np.array([[2, 3, 4], [1, 1, 1], [0, 2, -2]], np.float32)[:, None, :]
    g = np.array([[0, 0], [half, 0], [0, half]], np.float32)[:, None, :]
    beta = np.array([[1], [0.5], [1]], np.float32)
    s0 = np.array([[1, 0, 2], [0, 1, 0]], np.float32)[None, None]
    o, s = run(q, k, v, g, beta, initial_state=s0)
    want_o = np.array([[2, 4, 4], [2, 3.5, 3], [0.75, 1, 1.75]])
    want_s = np.array([[0.6875, 2, 0.4375], [-0.0625, 1, -1.3125]])
    assert np.max(np.abs(o[:, 0] - want_o)) < 1e-7, o[:, 0]
    assert np.max(np.abs(s[0, 0] - want_s)) < 1e-7, s[0, 0]


def check_explicit_matrices(run, seed=0):
    """Oracle equals the explicit K x K transition products on tiny random inputs."""
    rng = np.random.default_rng(seed)
    for T, K, V in ((1, 1, 1), (5, 3, 2), (8, 4, 3), (7, 2, 4), (8, 4, 4)):
        for with_state in (False, True):
            q, k, v, g, beta, s0 = _rand_case(rng, T, K, V, with_state)
            o, s = run(q, k, v, g, beta, initial_state=s0)
            ro, rs = reference.explicit_matrices(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0],
                                                 None if s0 is None else s0[0, 0])
            assert np.max(np.abs(o[:, 0] - ro)) <= 1e-13 * max(1.0, np.max(np.abs(ro)))
            assert np.max(np.abs(s[0, 0] - rs)) <= 1e-13 * max(1.0, np.max(np.abs(rs)))


def check_identity_when_no_write_no_decay(run, seed=1):
    """beta = 0 and g = 0 (alpha = 1): the state is untouched and o_t = S0^T q_t."""
    rng = np.random.default_rng(seed)
    T, K, V = 9, 5, 3
    q, k, v, _, _, s0 = _rand_case(rng, T, K, V)
    g = np.zeros((T, 1, K), np.float32)
    beta = np.zeros((T, 1), np.float32)
    o, s = run(q, k, v, g, beta, initial_state=s0)
    assert np.array_equal(s[0, 0], s0[0, 0].astype(np.float64))
    want = q[:, 0].astype(np.float64) @ s0[0, 0].astype(np.float64)
    assert np.max(np.abs(o[:, 0] - want)) <= 1e-14


def check_unit_key_overwrite(run, seed=2):
    """beta = 1 and |k| = 1 exactly: after the write S^T k = v. Keys use entries
    +-1/4 on 16 channels (exactly unit norm in binary floating point); q = k
    reads S^T k through the output."""
    rng = np.random.default_rng(seed)
    T, K, V = 12, 32, 5
    k = np.zeros((T, 1, K), np.float32)
    for t in range(T):
        idx = rng.choice(K, 16, replace=False)
        k[t, 0, idx] = rng.choice([-0.25, 0.25], 16)
    v = rng.standard_normal((T, 1, V)).astype(np.float32)
    g = (-0.2 * rng.random((T, 1, K))).astype(np.float32)
    beta = np.ones((T, 1), np.float32)
    s0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    o, _ = run(k.copy(), k, v, g, beta, initial_state=s0)
    assert np.max(np.abs(o[:, 0] - v[:, 0])) <= 1e-12


def check_basis_key_closed_form(run, seed=3):
    """Keys are basis vectors e_j: the write touches row j only,
    S[j] <- S'[j] + beta (v - S'[j]) with S' the decayed state; other rows only decay."""
    rng = np.random.default_rng(seed)
    T, K, V = 20, 6, 4
    j = rng.integers(0, K, T)
    k = np.zeros((T, 1, K), np.float32)
    k[np.arange(T), 0, j] = 1.0
    q = rng.standard_normal((T, 1, K)).astype(np.float32)
    v = rng.standard_normal((T, 1, V)).astype(np.float32)
    g = (-0.3 * rng.random((T, 1, K))).astype(np.float32)
    beta = rng.random((T, 1)).astype(np.float32)
    s0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    o, s = run(q, k, v, g, beta, initial_state=s0)
    S = s0[0, 0].astype(np.float64).copy()
    for t in range(T):
        for c in range(K):
            S[c] = S[c] * math.exp(float(g[t, 0, c]))
        b = float(beta[t, 0])
        S[j[t]] = (1.0 - b) * S[j[t]] + b * v[t, 0].astype(np.float64)
        want = np.zeros(V)
        for c in range(K):
            want += float(q[t, 0, c]) * S[c]
        assert np.max(np.abs(o[t, 0] - want)) <= 1e-12
    assert np.max(np.abs(s[0, 0] - S)) <= 1e-12


def check_chunked_equals_sequential(run, seed=4):
    """The chunked form equals the oracle for C in {1, 4, 16, 64}, partial last
    chunks and several in-chunk reference tokens."""
    rng = np.random.default_rng(seed)
    T, K, V = 37, 8, 6
    q, k, v, g, beta, s0 = _rand_case(rng, T, K, V)
    o, s = run(q, k, v, g, beta, initial_state=s0)
    scale = max(np.max(np.abs(o)), 1.0)
    for C in (1, 4, 16, 64):
        for ref in (0, C // 2, C - 1):
            co, cs = reference.chunked(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], s0[0, 0],
                                       chunk=C, ref=ref)
            assert np.max(np.abs(co - o[:, 0])) <= 1e-10 * scale
            assert np.max(np.abs(cs - s[0, 0])) <= 1e-10 * max(np.max(np.abs(cs)), 1.0)


def check_linear_in_values_and_state(run, seed=5):
    """With q, k, g, beta fixed, (o, S_T) is linear in (v, S0)."""
    rng = np.random.default_rng(seed)
    T, K, V = 15, 5, 4
    q, k, v1, g, beta, s1 = _rand_case(rng, T, K, V)
    # values on a 1/256 grid, so v1 + 2 v2 and s1 + 2 s2 are exact in fp32
    v1, s1 = (np.round(x * 256) / 256 for x in (v1, s1))
    v2 = np.round(rng.standard_normal(v1.shape) * 256) / 256
    s2 = np.round(rng.standard_normal(s1.shape) * 256) / 256
    v1, v2, s1, s2 = (x.astype(np.float32) for x in (v1, v2, s1, s2))
    o1, f1 = run(q, k, v1, g, beta, initial_state=s1)
    o2, f2 = run(q, k, v2, g, beta, initial_state=s2)
    o3, f3 = run(q, k, v1 + 2 * v2, g, beta, initial_state=s1 + 2 * s2)
    assert np.max(np.abs(o3 - (o1 + 2 * o2))) <= 1e-12
    assert np.max(np.abs(f3 - (f1 + 2 * f2))) <= 1e-12


def check_value_column_independence(run, seed=6):
    """Column j of o and S depends only on column j of v and S0."""
    rng = np.random.default_rng(seed)
    T, K, V = 11, 4, 6
    q, k, v, g, beta, s0 = _rand_case(rng, T, K, V)
    perm = rng.permutation(V)
    o, s = run(q, k, v, g, beta, initial_state=s0)
    po, ps = run(q, k, v[:, :, perm], g, beta, initial_state=s0[..., perm])
    assert np.max(np.abs(po - o[:, :, perm])) <= 1e-13
    assert np.max(np.abs(ps - s[..., perm])) <= 1e-13


ALL_CHECKS = [
    check_hand_example,
    check_explicit_matrices,
    check_identity_when_no_write_no_decay,
    check_unit_key_overwrite,
    check_basis_key_closed_form,
    check_chunked_equals_sequential,
    check_linear_in_values_and_state,
    check_value_column_independence,
]


# ---------------------------------------------------------------------------
# Backward: each check takes a function with the signature of oracle.backward.

_GRADS = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def _bwd_case(rng, T, H, K, V, N=1, scalar_gate=False):
    q = rng.standard_normal((T, H, K)).astype(np.float32)
    k = (rng.standard_normal((T, H, K)) / math.sqrt(K)).astype(np.float32)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    gshape = (T, H) if scalar_gate else (T, H, K)
    g = (-0.4 * rng.random(gshape)).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    s0 = (rng.standard_normal((N, H, K, V)) * 0.5).astype(np.float32)
    do = rng.standard_normal((T, H, V)).astype(np.float32)
    dsT = rng.standard_normal((N, H, K, V)).astype(np.float32)
    return q, k, v, g, beta, s0, do, dsT


def _fd_loss(q, k, v, g, beta, s0, do, dsT, cu):
    """L = sum <dO, o> + <dS_T, S_T> from the explicit K x K transition products (fp64)."""
    T, H, K = q.shape
    if g.ndim == 2:
        g = np.broadcast_to(g[:, :, None], (T, H, K))
    total = 0.0
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        for h in range(H):
            o, S = reference.explicit_matrices(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h],
                                               beta[a:b, h], s0[n, h])
            total += np.sum(o * do[a:b, h]) + np.sum(S * dsT[n, h])
    return total


def _check_fd(run_bwd, case, cu, tol=1e-7):
    q, k, v, g, beta, s0, do, dsT = case
    got = run_bwd(q, k, v, g, beta, do, cu_seqlens=cu, initial_state=s0, d_final_state=dsT)
    args = [x.astype(np.float64) for x in (q, k, v, g, beta, s0)]
    eps = 1e-6
    for ai, name in enumerate(_GRADS):
        fd = np.zeros_like(args[ai])
        for idx in np.ndindex(args[ai].shape):
            up = [x.copy() for x in args]
            dn = [x.copy() for x in args]
            up[ai][idx] += eps
            dn[ai][idx] -= eps
            fd[idx] = (_fd_loss(*up, do, dsT, cu) - _fd_loss(*dn, do, dsT, cu)) / (2 * eps)
        err = np.max(np.abs(fd - got[name]))
        assert err <= tol * max(1.0, np.max(np.abs(fd))), (name, err)


def check_bwd_finite_differences(run_bwd, seed=20):
    """Every gradient equals central finite differences (fp64, step 1e-6) of the
    loss computed from the explicit transition products: two packed sequences of
    two heads, with initial states and a final-state gradient."""
    rng = np.random.default_rng(seed)
    _check_fd(run_bwd, _bwd_case(rng, 9, 2, 3, 2, N=2), np.array([0, 4, 9]))


def check_bwd_finite_differences_scalar_gate(run_bwd, seed=21):
    """As above for a [T, H] gate (one decay per token and head)."""
    rng = np.random.default_rng(seed)
    _check_fd(run_bwd, _bwd_case(rng, 7, 1, 3, 2, scalar_gate=True), np.array([0, 7]))


def check_bwd_finite_differences_long(run_bwd, seed=22):
    """A 70-token sequence (the state is recomputed block by block in the reverse
    pass): finite differences again, on K = V = 2."""
    rng = np.random.default_rng(seed)
    case = list(_bwd_case(rng, 70, 1, 2, 2))
    case[3] = (-0.05 * rng.random((70, 1, 2))).astype(np.float32)  # keep the state alive
    _check_fd(run_bwd, tuple(case), np.array([0, 70]), tol=1e-6)


def check_bwd_no_write_closed_form(run_bwd, seed=23):
    """beta = 0: S_t = Diag(exp(G_t)) S0 with G_t = g_1 + ... + g_t, so with
    R_t = sum_{s >= t} Diag(exp(G_s - G_t)) q_s dO_s^T + Diag(exp(G_T - G_t)) dS_T
    (the gradient reaching S_t): dq_t = S_t dO_t, dk = dv = 0,
    dbeta_t = (R_t^T k_t) . (v_t - S_t^T k_t),
    dS0 = sum_s Diag(exp(G_s)) q_s dO_s^T + Diag(exp(G_T)) dS_T, and
    dg_t[c] = sum_{s >= t} exp(G_s[c]) q_s[c] (S0 dO_s)[c] + exp(G_T[c]) sum_j S0[c,j] dS_T[c,j]."""
    rng = np.random.default_rng(seed)
    T, K, V = 12, 4, 3
    q, k, v, g, _, s0, do, dsT = _bwd_case(rng, T, 1, K, V)
    beta = np.zeros((T, 1), np.float32)
    got = run_bwd(q, k, v, g, beta, do, initial_state=s0, d_final_state=dsT)
    q64, k64, v64, g64, do64 = (x[:, 0].astype(np.float64) for x in (q, k, v, g, do))
    S0, dST = s0[0, 0].astype(np.float64), dsT[0, 0].astype(np.float64)
    G = np.cumsum(g64, axis=0)
    for t in range(T):
        St = np.exp(G[t])[:, None] * S0
        R = np.exp(G[-1] - G[t])[:, None] * dST
        for s in range(t, T):
            R += np.exp(G[s] - G[t])[:, None] * np.outer(q64[s], do64[s])
        assert np.allclose(got["dq"][t, 0], St @ do64[t], rtol=0, atol=1e-12)
        want_db = (R.T @ k64[t]) @ (v64[t] - St.T @ k64[t])
        assert abs(got["dbeta"][t, 0] - want_db) <= 1e-11 * max(1.0, abs(want_db))
        want_dg = np.exp(G[-1]) * np.sum(S0 * dST, axis=1)
        for s in range(t, T):
            want_dg += np.exp(G[s]) * q64[s] * (S0 @ do64[s])
        assert np.allclose(got["dg"][t, 0], want_dg, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(got["dk"])) == 0.0 and np.max(np.abs(got["dv"])) == 0.0
    want_ds0 = np.exp(G[-1])[:, None] * dST
    for s in range(T):
        want_ds0 += np.exp(G[s])[:, None] * np.outer(q64[s], do64[s])
    assert np.allclose(got["d_initial_state"][0, 0], want_ds0, rtol=1e-12, atol=1e-12)


def check_bwd_homogeneity(run_bwd, seed=24):
    """Euler's identity for maps homogeneous of degree one: o is linear in q, and
    (o, S_T) is jointly linear in (v, S0), so with L = <dO, o> + <dS_T, S_T>,
    <dq, q> = <dO, o> and <dv, v> + <dS0, S0> = L (packed sequences, 3 heads)."""
    rng = np.random.default_rng(seed)
    lens = [20, 1, 37]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, s0, do, dsT = _bwd_case(rng, sum(lens), 3, 6, 5, N=len(lens))
    got = run_bwd(q, k, v, g, beta, do, cu_seqlens=cu, initial_state=s0, d_final_state=dsT)
    o = np.zeros(do.shape)
    fs = np.zeros(s0.shape)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        for h in range(3):
            o[a:b, h], fs[n, h] = reference.explicit_matrices(q[a:b, h], k[a:b, h], v[a:b, h],
                                                              g[a:b, h], beta[a:b, h], s0[n, h])
    lo = np.sum(o * do)
    L = lo + np.sum(fs * dsT)
    assert abs(np.sum(got["dq"] * q) - lo) <= 1e-11 * max(1.0, abs(lo))
    lhs = np.sum(got["dv"] * v) + np.sum(got["d_initial_state"] * s0)
    assert abs(lhs - L) <= 1e-11 * max(1.0, abs(L))


def check_bwd_empty_sequence_passes_state_gradient(run_bwd, seed=25):
    """A sequence of length 0 leaves its state unchanged, so dS0 = dS_T for it."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, s0, do, dsT = _bwd_case(rng, 5, 2, 3, 2, N=3)
    got = run_bwd(q, k, v, g, beta, do, cu_seqlens=np.array([0, 2, 2, 5]), initial_state=s0,
                  d_final_state=dsT)
    assert np.array_equal(got["d_initial_state"][1], dsT[1].astype(np.float64))


BACKWARD_CHECKS = [
    check_bwd_finite_differences,
    check_bwd_finite_differences_scalar_gate,
    check_bwd_finite_differences_long,
    check_bwd_no_write_closed_form,
    check_bwd_homogeneity,
    check_bwd_empty_sequence_passes_state_gradient,
]
