"""Pins of the oracle's gated and delta-rule recurrences.

GLA: S_t = diag(alpha_t) S_{t-1} + k_t v_t^T ("Linear Attention", GLA);
gated delta rule: S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T
("Story of Attention Part 5", section 7), o_t = S_t^T q_t, S feature-major.
Pinned to: the printed d = 2 worked example; the gradient-descent reading the
page gives (one step of size beta on 1/2 |S^T k - v|^2, by finite
differences); the erase/write product form the page expands; exact overwrite
of orthonormal keys; pure decay when nothing is written; and, for GLA,
explicit pairwise sums with products of gates and the retention oracle
(itself pinned to its own worked example) for a constant scalar gate.
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def test_delta_rule_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "t5_delta_rule_worked_example.json")))
    k = np.array(g["k"], float)
    v = np.array(g["v"], float)
    S_prev = np.array(g["S_prev"], float).T  # feature-major: row = key component
    Q = k.reshape(1, 1, 1, 2)  # query with the same key
    O, S = oracle.delta_recurrent(Q, k.reshape(1, 1, 1, 2), v.reshape(1, 1, 1, 2), np.full((1, 1, 1), g["beta"]),
                                  S_in=S_prev.reshape(1, 1, 2, 2))
    np.testing.assert_array_equal(S_prev.T @ k, g["prediction"])
    np.testing.assert_array_equal(S[0, 0].T, np.array(g["S_new"], float))
    np.testing.assert_array_equal(O[0, 0, 0], v)  # the new state returns exactly v for k


def test_delta_step_is_one_gradient_step():
    # S_t = S' - beta grad L(S') with S' = alpha S_{t-1}, L(S) = 1/2 |S^T k - v|^2
    rng = _rng(1)
    dk, dv = 5, 3
    S0 = rng.standard_normal((dk, dv))
    k, v, q = rng.standard_normal(dk), rng.standard_normal(dv), rng.standard_normal(dk)
    for alpha, beta in ((None, 0.7), (0.8, 0.3)):
        a = 1.0 if alpha is None else alpha
        Sp = a * S0
        L = lambda S: 0.5 * float(((S.T @ k - v) ** 2).sum())  # noqa: E731
        grad = np.empty_like(Sp)
        h = 1e-6
        for idx in np.ndindex(*Sp.shape):
            e = np.zeros_like(Sp)
            e[idx] = h
            grad[idx] = (L(Sp + e) - L(Sp - e)) / (2 * h)
        want = Sp - beta * grad
        _, S = oracle.delta_recurrent(q.reshape(1, 1, 1, dk), k.reshape(1, 1, 1, dk), v.reshape(1, 1, 1, dv),
                                      np.full((1, 1, 1), beta),
                                      alpha=None if alpha is None else np.full((1, 1, 1), alpha),
                                      S_in=S0.reshape(1, 1, dk, dv))
        np.testing.assert_allclose(S[0, 0], want, rtol=1e-8, atol=1e-9)


def test_delta_rule_erase_write_form():
    # alpha = 1: S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t
    rng = _rng(2)
    B, H, N, dk, dv = 1, 2, 9, 4, 3
    Q, K = rng.standard_normal((B, H, N, dk)), rng.standard_normal((B, H, N, dk)) / 2
    V = rng.standard_normal((B, H, N, dv))
    beta = rng.uniform(0, 1, (B, H, N))
    S_in = rng.standard_normal((B, H, dk, dv))
    O, S = oracle.delta_recurrent(Q, K, V, beta, S_in=S_in)
    for h in range(H):
        St = S_in[0, h].copy()
        for t in range(N):
            kt = K[0, h, t]
            St = (np.eye(dk) - beta[0, h, t] * np.outer(kt, kt)) @ St + beta[0, h, t] * np.outer(kt, V[0, h, t])
            np.testing.assert_allclose(O[0, h, t], St.T @ Q[0, h, t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, rtol=1e-12, atol=1e-12)


def test_delta_rule_overwrites_orthonormal_keys():
    rng = _rng(3)
    d = 6
    Kb = np.linalg.qr(rng.standard_normal((d, d)))[0].T  # orthonormal rows
    vals = rng.standard_normal((2 * d, d))
    order = list(range(d)) + [2, 4]  # every key once, then keys 2 and 4 again with new values
    K = np.stack([Kb[i] for i in order])[None, None]
    V = vals[:len(order)][None, None]
    _, S = oracle.delta_recurrent(K, K, V, np.ones((1, 1, len(order))))
    last = {i: V[0, 0, j] for j, i in enumerate(order)}
    for i in range(d):
        np.testing.assert_allclose(S[0, 0].T @ Kb[i], last[i], atol=1e-12)


def test_gated_delta_pure_decay_when_nothing_is_written():
    rng = _rng(4)
    B, H, N, dk, dv = 1, 1, 7, 3, 2
    Q = rng.standard_normal((B, H, N, dk))
    K = rng.standard_normal((B, H, N, dk))
    V = rng.standard_normal((B, H, N, dv))
    alpha = rng.uniform(0.5, 1.0, (B, H, N))
    S_in = rng.standard_normal((B, H, dk, dv))
    O, S = oracle.delta_recurrent(Q, K, V, np.zeros((B, H, N)), alpha=alpha, S_in=S_in)
    cum = np.cumprod(alpha[0, 0])
    for t in range(N):
        np.testing.assert_allclose(O[0, 0, t], cum[t] * S_in[0, 0].T @ Q[0, 0, t], rtol=1e-13)
    np.testing.assert_allclose(S[0, 0], cum[-1] * S_in[0, 0], rtol=1e-13)


def test_gla_matches_pairwise_sums_with_gate_products():
    rng = _rng(5)
    B, H, N, dk, dv = 2, 1, 8, 3, 4
    Q, K, V = rng.standard_normal((B, H, N, dk)), rng.standard_normal((B, H, N, dk)), rng.standard_normal((B, H, N, dv))
    A = rng.uniform(0.3, 1.0, (B, H, N, dk))
    S_in = rng.standard_normal((B, H, dk, dv))
    O, S = oracle.gla_recurrent(Q, K, V, A, S_in=S_in)
    for b in range(B):
        a = A[b, 0]
        for t in range(N):
            # gate product over (s, t]: prod_{r=s+1..t} a_r, channel-wise
            want = (Q[b, 0, t] * np.prod(a[:t + 1], axis=0)) @ S_in[b, 0]
            for s in range(t + 1):
                g = np.prod(a[s + 1:t + 1], axis=0)
                want = want + float((Q[b, 0, t] * g * K[b, 0, s]).sum()) * V[b, 0, s]
            np.testing.assert_allclose(O[b, 0, t], want, rtol=1e-12, atol=1e-12)


def test_gla_constant_gate_is_retention():
    rng = _rng(6)
    B, H, N, d = 1, 3, 20, 4
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    gam = np.array([0.5, 0.9, 1.0])
    A = np.broadcast_to(gam[None, :, None, None], (B, H, N, d)).copy()
    O, S = oracle.gla_recurrent(Q, K, V, A)
    Or, Sr = oracle.retention_recurrent("identity", Q, K, V, gam)
    np.testing.assert_allclose(O, Or, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sr, rtol=1e-12, atol=1e-12)
