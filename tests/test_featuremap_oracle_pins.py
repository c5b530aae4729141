"""Pins of the oracle's further feature maps ("Linear Attention" (aiwiki.ai),
feature-map table: DPFP, cosine / sine projections; "Story of Attention Part
5", section 3: cosFormer).

cosFormer is pinned to the printed worked example (every printed matrix) and
to explicit pairwise sums with the cosine weight of the position difference
(causal, with a starting state carried across a split, where positions must
continue).  DPFP is pinned to hand-computed vectors and to its kernel written
as products of ReLU shifts of both inputs.  The cos/sin projections are pinned
by cos(a)cos(b) + sin(a)sin(b) = cos(a - b) and by W = 0 (every weight 1: a
running mean of V).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _reset_map():
    yield
    oracle.set_map(0, 0)


def _t6():
    with open(os.path.join(GOLDEN, "t6_cosformer_worked_example.json")) as f:
        g = json.load(f)
    Q, K, V = (np.array(g[n], float)[None, None] for n in ("Q", "K", "V"))
    return g, Q, K, V


def test_cosformer_worked_example_every_printed_matrix():
    g, Q, K, V = _t6()
    M, dec = g["M"], g["decimals"]
    oracle.set_map(M, 0)
    fq, fk = oracle.phi("cosformer", Q[0, 0]), oracle.phi("cosformer", K[0, 0])
    d = 4
    # the map's first half at position 0 is ReLU(x) (cos 0 = 1, sin 0 = 0)
    np.testing.assert_array_equal(fq[0, :d], g["phiQ"][0])
    np.testing.assert_array_equal(fk[0, :d], g["phiK"][0])
    relu_q, relu_k = np.maximum(Q[0, 0], 0), np.maximum(K[0, 0], 0)
    np.testing.assert_array_equal(relu_q, g["phiQ"])
    np.testing.assert_array_equal(relu_k, g["phiK"])
    np.testing.assert_array_equal(relu_q @ relu_k.T, g["base_scores"])
    # phi(q_i) . phi(k_j) = base_ij * C_ij: the printed reweighted scores
    np.testing.assert_array_equal(np.round(fq @ fk.T, dec), g["B_cos"])
    np.testing.assert_array_equal(np.round((fq @ fk.T) / (relu_q @ relu_k.T + (relu_q @ relu_k.T == 0)), dec)
                                  [relu_q @ relu_k.T > 0], np.array(g["C"])[relu_q @ relu_k.T > 0])
    O, S, z = oracle.noncausal("cosformer", Q, K, V)
    np.testing.assert_array_equal(np.round(O[0, 0], dec), g["output"])
    num, den = oracle.state_read(fq, S[0, 0], z[0, 0])
    np.testing.assert_array_equal(np.round((fq @ fk.T) / den[:, None], dec), g["A_cos"])


@pytest.mark.parametrize("M,pos0", [(4, 0), (50, 0), (300, 17)])
def test_cosformer_causal_equals_cosine_weighted_pairs(M, pos0):
    rng = np.random.default_rng(M)
    B, H, N, d = 1, 2, 40, 3
    Q, K, V = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, 2))
    Q[..., 0] = np.abs(Q[..., 0]) + 0.1  # every ReLU(q) nonzero: no 0/0 rows
    K[..., 0] = np.abs(K[..., 0]) + 0.1
    oracle.set_map(M, pos0)
    O, S, z = oracle.causal_recurrent("cosformer", Q, K, V)
    Oc, Sc, zc = oracle.causal_chunked("cosformer", Q, K, V, 7)
    for h in range(H):
        rq, rk = np.maximum(Q[0, h], 0), np.maximum(K[0, h], 0)
        for i in range(N):
            w = np.array([rq[i] @ rk[j] * np.cos(np.pi * (i - j) / (2 * M)) for j in range(i + 1)])
            want = w @ V[0, h, :i + 1] / w.sum()
            np.testing.assert_allclose(O[0, h, i], want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Oc, O, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-11, atol=1e-12)
    # a split at t: the second call starts at position pos0 + t with the first call's state
    t = 13
    _, S1, z1 = oracle.causal_recurrent("cosformer", Q[:, :, :t], K[:, :, :t], V[:, :, :t])
    oracle.set_map(M, pos0 + t)
    O2, S2, _ = oracle.causal_recurrent("cosformer", Q[:, :, t:], K[:, :, t:], V[:, :, t:], S_in=S1, z_in=z1)
    np.testing.assert_allclose(O2, O[:, :, t:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-11, atol=1e-12)


def test_dpfp_hand_computed():
    # x = [1, 2]: r = ReLU([1, 2, -1, -2]) = [1, 2, 0, 0];
    # nu = 1: r_j r_{j+1} = [2, 0, 0, 0]; nu = 2 adds r_j r_{j+2} = [0, 0, 0, 0]
    oracle.set_map(2, 0)
    np.testing.assert_array_equal(oracle.phi("dpfp", np.array([[1.0, 2.0]])), [[2, 0, 0, 0, 0, 0, 0, 0]])
    # x = [3, -1]: r = [3, 0, 0, 1]; shift 1: [0, 0, 0, 3]; shift 2: [0, 0, 0, 0]
    np.testing.assert_array_equal(oracle.phi("dpfp", np.array([[3.0, -1.0]])), [[0, 0, 0, 3, 0, 0, 0, 0]])
    # x = [-2, 5]: r = [0, 5, 2, 0]; shift 1: [0, 10, 0, 0]; shift 2: [0, 0, 0, 0]
    np.testing.assert_array_equal(oracle.phi("dpfp", np.array([[-2.0, 5.0]])), [[0, 10, 0, 0, 0, 0, 0, 0]])


def test_dpfp_kernel_is_products_of_shifted_relus():
    rng = np.random.default_rng(3)
    d, nu = 5, 3
    oracle.set_map(nu, 0)
    for _ in range(10):
        x, y = rng.standard_normal(d), rng.standard_normal(d)
        rx, ry = np.maximum(np.r_[x, -x], 0), np.maximum(np.r_[y, -y], 0)
        want = sum(float((rx * np.roll(rx, -i) * ry * np.roll(ry, -i)).sum()) for i in range(1, nu + 1))
        fx, fy = oracle.phi("dpfp", x[None]), oracle.phi("dpfp", y[None])
        assert fx.shape == (1, 2 * d * nu)
        assert (fx >= 0).all()
        np.testing.assert_allclose((fx @ fy.T)[0, 0], want, rtol=1e-13)


def test_trig_features_kernel_identity_and_zero_projection():
    rng = np.random.default_rng(4)
    m, d = 7, 3
    W = rng.standard_normal((m, d))
    x, y = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    fx, fy = oracle.phi("trig", x, W), oracle.phi("trig", y, W)
    assert fx.shape == (1, 2 * m)
    np.testing.assert_allclose((fx @ fy.T)[0, 0], np.cos(W @ (x[0] - y[0])).sum(), rtol=1e-13)
    # W = 0: every feature vector is [1..1, 0..0], all weights equal: causal running mean of V
    B, H, N = 1, 1, 9
    Q, K, V = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, 2))
    O, _, _ = oracle.causal_recurrent("trig", Q, K, V, np.zeros((m, d)))
    np.testing.assert_allclose(O[0, 0], np.cumsum(V[0, 0], 0) / np.arange(1, N + 1)[:, None], rtol=1e-13)
