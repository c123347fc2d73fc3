"""NumPy fp64 forms of KDA prefill used to pin the C oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both functions work on one sequence of one head: q, k, g [T, K]; v [T, V];
beta [T]; S0 [K, V] or None. They return (o [T, V], S_T [K, V]).

* :func:`explicit_matrices` multiplies out the K x K transition of every token,
  S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T with
  alpha_t = exp(g_t), o_t = S_t^T q_t. It builds the matrices instead of using
  the rank-1 update the C oracle uses, so a slip in either shows up as a
  mismatch. Meant for tiny K.

* :func:`chunked` is the chunk-parallel form: the sequence is cut into chunks
  of C tokens (augursoft.site "Kimi K3 的三個系統設計", section
  "為什麼 FlashKDA 選擇 16-token chunks", where the chunk is 16 tokens and a 16 x 16
  matrix inversion appears). Inside a chunk, with G the running sum of g from
  the chunk start, the delta-rule writes form a unit lower triangular system
  (I + A) Delta = diag(beta) (V - K+ S0), solved by the inverse T = (I + A)^-1;
  the outputs and the end-of-chunk state then follow from matrix products.
  The derivation is in the function body. In exact arithmetic it equals the
  token-by-token recurrence for every chunk size and every reference point.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def explicit_matrices(q, k, v, g, beta, S0=None):
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, K = k.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if S0 is None else _f64(S0).copy()
    eye = np.eye(K)
    o = np.zeros((T, V))
    for t in range(T):
        decay = np.diag(np.exp(g[t]))
        keep = eye - beta[t] * np.outer(k[t], k[t])
        S = keep @ decay @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def chunked(q, k, v, g, beta, S0=None, chunk=16, ref=None, intermediates=False):
    """Chunked evaluation; ``ref`` is the in-chunk token whose cumulative gate
    is factored out of the in-chunk products (default: the middle token).

    Derivation. Let D_r = Diag(exp(G_r)) with G_r = g_1 + ... + g_r inside the
    chunk and S_0 the state at the chunk start. Unrolling the recurrence,
        S_r = D_r (S_0 + sum_{i<=r} (k_i * exp(-G_i)) delta_i^T),
        delta_i = beta_i (v_i - S_{i-1}'^T k_i),  S_{i-1}' = Diag(exp(g_i)) S_{i-1},
    and S_{i-1}'^T k_i = S_0^T K+_i + sum_{j<i} (k_i . (k_j * exp(G_i - G_j))) delta_j
    with K+_i = k_i * exp(G_i). Stacking the delta_i:
        (I + A) Delta = diag(beta) (V - K+ S_0),
        A[r, i] = beta_r sum_c k[r,c] k[i,c] exp(G[r,c] - G[i,c])   (i < r),
    so Delta = U - W S_0 with T = (I + A)^-1, U = T diag(beta) V,
    W = T diag(beta) K+. Then
        o_r = S_r^T q_r = Q+_r^T S_0 + sum_{i<=r} P[r, i] delta_i,
        P[r, i] = sum_c q[r,c] k[i,c] exp(G[r,c] - G[i,c])          (i <= r),
        S_C = Diag(gamma) S_0 + K^d^T Delta,  gamma = exp(G_C),  K^d_i = k_i * exp(G_C - G_i).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, K = k.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if S0 is None else _f64(S0).copy()
    o = np.zeros((T, V))
    inter = []
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        n = c1 - c0
        qc, kc, vc, gc, bc = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1]
        G = np.cumsum(gc, axis=0)
        r = (n // 2) if ref is None else min(ref, n - 1)
        Gref = G[r]
        k_hat = kc * np.exp(G - Gref)
        q_hat = qc * np.exp(G - Gref)
        k_rev = kc * np.exp(Gref - G)
        A = np.tril(bc[:, None] * (k_hat @ k_rev.T), -1)
        P = np.tril(q_hat @ k_rev.T, 0)
        Tinv = np.linalg.inv(np.eye(n) + A)
        k_plus = kc * np.exp(G)
        q_plus = qc * np.exp(G)
        k_d = kc * np.exp(G[-1] - G)
        gamma = np.exp(G[-1])
        W = Tinv @ (bc[:, None] * k_plus)
        U = Tinv @ (bc[:, None] * vc)
        Delta = U - W @ S
        o[c0:c1] = q_plus @ S + P @ Delta
        if intermediates:
            inter.append(dict(G=G, A=A, P=P, T=Tinv, W=W, U=U, Qp=q_plus, Kd=k_d,
                              gamma=gamma, S0=S.copy(), Delta=Delta))
        S = gamma[:, None] * S + k_d.T @ Delta
    if intermediates:
        return o, S, inter
    return o, S


def chunked_backward(q, k, v, g, beta, dO, S0=None, dST=None, chunk=16, ref=None, intermediates=False):
    """Gradients of L = <dO, o> + <dS_T, S_T> through the chunked form above.

    One sequence of one head (shapes as :func:`chunked`, dO [T, V], dST [K, V]).
    Returns dict(dq, dk, dv, dg, dbeta, dS0), plus with ``intermediates`` the lists
    S0s (each chunk's start state) and Rs (the gradient reaching each chunk's end
    state), in chunk order. The reverse pass runs over chunks;
    R is the gradient reaching the chunk's end state. With the chunk's start
    state S0 and U = V - K+ S0, Delta = T diag(beta) U:
        dDelta = P^T dO + K^d R,      dU = (T diag(beta))^T dDelta,    dv = dU,
        dQ+ = dO S0^T,  dK+ = -dU S0^T,  dK^d = Delta R^T,  dgamma = rowsum(R * S0),
        dP = tril(dO Delta^T),  d(T diag(beta)) = dDelta U^T,
        R <- Diag(gamma) R + Q+^T dO - K+^T dU   (the gradient reaching S0).
    The triangular inverse gives dA = -T^T dT T^T (strictly lower part), and A,
    P, K+, Q+, K^d, gamma pass their gradients to q, k, beta and the running
    gate G, whose reverse running sum inside the chunk is dg. The reference
    token factored out of A and P (as in :func:`chunked`) cancels in every
    product, so no gradient flows through it.
    """
    q, k, v, g, beta, dO = map(_f64, (q, k, v, g, beta, dO))
    T, K = k.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if S0 is None else _f64(S0).copy()
    starts = []
    for c0 in range(0, T, chunk):
        starts.append(S.copy())
        _, S = chunked(q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk], g[c0:c0 + chunk],
                       beta[c0:c0 + chunk], S, chunk=chunk, ref=ref)
    R = np.zeros((K, V)) if dST is None else _f64(dST).copy()
    dq, dk, dg = np.zeros((T, K)), np.zeros((T, K)), np.zeros((T, K))
    dv, dbeta = np.zeros((T, V)), np.zeros(T)
    ends = [None] * len(starts)
    for ci in range(len(starts) - 1, -1, -1):
        ends[ci] = R.copy()
        c0 = ci * chunk
        c1 = min(c0 + chunk, T)
        n = c1 - c0
        qc, kc, vc, gc, bc, D = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1], dO[c0:c1]
        S0c = starts[ci]
        G = np.cumsum(gc, axis=0)
        r = (n // 2) if ref is None else min(ref, n - 1)
        up, dn = np.exp(G - G[r]), np.exp(G[r] - G)
        k_hat, q_hat, k_rev = kc * up, qc * up, kc * dn
        KK = k_hat @ k_rev.T
        A = np.tril(bc[:, None] * KK, -1)
        P = np.tril(q_hat @ k_rev.T, 0)
        Tinv = np.linalg.inv(np.eye(n) + A)
        Tb = Tinv * bc[None, :]
        Kp, Qp = kc * np.exp(G), qc * np.exp(G)
        Kd = kc * np.exp(G[-1] - G)
        gamma = np.exp(G[-1])
        U = vc - Kp @ S0c
        Delta = Tb @ U

        dDelta = P.T @ D + Kd @ R
        dU = Tb.T @ dDelta
        dv[c0:c1] = dU
        dQp = D @ S0c.T
        dKp = -dU @ S0c.T
        dKd = Delta @ R.T
        dgamma = np.sum(R * S0c, axis=1)
        dP = np.tril(D @ Delta.T, 0)
        dTb = dDelta @ U.T
        dbeta_c = np.sum(dTb * Tinv, axis=0)
        dT = dTb * bc[None, :]
        dA = np.tril(-Tinv.T @ dT @ Tinv.T, -1)
        dbeta_c += np.sum(dA * KK, axis=1)
        dAt = dA * bc[:, None]
        dk_hat = dAt @ k_rev
        dk_rev = dAt.T @ k_hat + dP.T @ q_hat
        dq_hat = dP @ k_rev

        dkc = dk_hat * up + dk_rev * dn + dKp * np.exp(G) + dKd * np.exp(G[-1] - G)
        dqc = dq_hat * up + dQp * np.exp(G)
        dG = dk_hat * k_hat - dk_rev * k_rev + dq_hat * q_hat + dKp * Kp + dQp * Qp - dKd * Kd
        dG[-1] += np.sum(dKd * Kd, axis=0) + dgamma * gamma
        dg[c0:c1] = np.cumsum(dG[::-1], axis=0)[::-1]
        dq[c0:c1], dk[c0:c1], dbeta[c0:c1] = dqc, dkc, dbeta_c
        R = gamma[:, None] * R + Qp.T @ D - Kp.T @ dU
    res = dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dS0=R)
    if intermediates:
        res["S0s"], res["Rs"] = starts, ends
    return res
