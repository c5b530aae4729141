"""Pins of the retention oracle (decayed, unnormalised linear attention).

The oracle's retention functions follow "Story of Attention Part 5",
section 4 (RetNet: parallel form (Q K^T (.) D) V, recurrent form
S_n = gamma S_{n-1} + k_n^T v_n, o_n = q_n S_n) and section 6 (Lightning
Attention blockwise form).  They are pinned here against the page's printed
worked example, against each other (three independent forms that the page
says compute one function), against closed forms at gamma = 0 and for a
single impulse, and against the separately pinned normalised oracle at
gamma = 1.  CPU only.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t4():
    with open(os.path.join(GOLDEN, "t4_retnet_worked_example.json")) as f:
        g = json.load(f)
    arr = {k: np.array(g[k], dtype=np.float64) for k in ("Q", "K", "V")}
    return g, arr["Q"].reshape(1, 1, 4, 4), arr["K"].reshape(1, 1, 4, 4), arr["V"].reshape(1, 1, 4, 4)


def test_t4_parallel_and_recurrent_outputs_equal_printed():
    g, Q, K, V = _t4()
    want = np.array(g["output_parallel"])
    par = oracle.retention_parallel("identity", Q, K, V, g["gamma"])[0, 0]
    rec, _ = oracle.retention_recurrent("identity", Q, K, V, g["gamma"])
    np.testing.assert_allclose(par, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rec[0, 0], want, rtol=0, atol=1e-12)
    # the page's recurrent check of token 3
    np.testing.assert_allclose(rec[0, 0, 2], np.array(g["output_3"]), rtol=0, atol=1e-12)


def test_t4_recurrent_states_equal_printed():
    g, Q, K, V = _t4()
    for n in (1, 2, 3):
        _, S = oracle.retention_recurrent("identity", Q[:, :, :n], K[:, :, :n], V[:, :, :n], g["gamma"])
        np.testing.assert_allclose(S[0, 0], np.array(g[f"S_{n}"]), rtol=0, atol=1e-12, err_msg=f"S_{n}")


@pytest.mark.parametrize("C", [1, 2, 3, 4])
def test_t4_blockwise_equals_printed(C):
    g, Q, K, V = _t4()
    O, S = oracle.retention_chunked("identity", Q, K, V, g["gamma"], C)
    np.testing.assert_allclose(O[0, 0], np.array(g["output_parallel"]), rtol=0, atol=1e-12)
    _, S4 = oracle.retention_recurrent("identity", Q, K, V, g["gamma"])
    np.testing.assert_allclose(S, S4, rtol=0, atol=1e-12)


def _rand(seed, B, H, N, d, dv):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)) / np.sqrt(d), rng.standard_normal((B, H, N, d)) / np.sqrt(d),
            rng.standard_normal((B, H, N, dv)))


@pytest.mark.parametrize("phi", ["identity", "elu1"])
@pytest.mark.parametrize("with_state", [False, True])
def test_parallel_recurrent_blockwise_agree(phi, with_state):
    B, H, N, d, dv = 2, 3, 37, 5, 4
    Q, K, V = _rand(7, B, H, N, d, dv)
    gam = np.array([0.3, 0.9, 1.0])
    S0 = np.random.default_rng(8).standard_normal((B, H, d, dv)) if with_state else None
    rec, Srec = oracle.retention_recurrent(phi, Q, K, V, gam, S_in=S0)
    par = oracle.retention_parallel(phi, Q, K, V, gam, S_in=S0)
    np.testing.assert_allclose(par, rec, rtol=1e-12, atol=1e-12)
    for C in (1, 2, 5, 8, 16, 36, 37, 64):
        blk, Sblk = oracle.retention_chunked(phi, Q, K, V, gam, C, S_in=S0)
        np.testing.assert_allclose(blk, rec, rtol=1e-11, atol=1e-11, err_msg=f"C={C}")
        np.testing.assert_allclose(Sblk, Srec, rtol=1e-11, atol=1e-11, err_msg=f"C={C}")


def test_favor_feature_map_with_decay_agrees():
    B, H, N, d, dv, m = 1, 2, 20, 4, 3, 12
    Q, K, V = _rand(9, B, H, N, d, dv)
    W = np.random.default_rng(10).standard_normal((m, d))
    rec, _ = oracle.retention_recurrent("favor", Q, K, V, [0.7, 0.95], W=W)
    blk, _ = oracle.retention_chunked("favor", Q, K, V, [0.7, 0.95], 6, W=W)
    np.testing.assert_allclose(blk, rec, rtol=1e-11, atol=1e-12)


def test_gamma_zero_keeps_only_the_diagonal():
    """gamma = 0: D is the identity, so o_i = (q_i . k_i) v_i."""
    Q, K, V = _rand(11, 1, 1, 9, 4, 3)
    rec, _ = oracle.retention_recurrent("identity", Q, K, V, 0.0)
    want = np.einsum("bhnd,bhnd->bhn", Q, K)[..., None] * V
    np.testing.assert_allclose(rec, want, rtol=1e-13, atol=1e-14)
    blk, _ = oracle.retention_chunked("identity", Q, K, V, 0.0, 4)
    np.testing.assert_allclose(blk, want, rtol=1e-13, atol=1e-14)


def test_single_impulse_decays_geometrically():
    """Only token 0 carries a value: o_i = gamma^i (q_i . k_0) v_0."""
    Q, K, V = _rand(12, 1, 1, 12, 3, 2)
    V[:, :, 1:] = 0.0
    g = 0.8
    rec, _ = oracle.retention_recurrent("identity", Q, K, V, g)
    qk0 = (Q[0, 0] @ K[0, 0, 0])
    want = (g ** np.arange(12) * qk0)[:, None] * V[0, 0, 0][None, :]
    np.testing.assert_allclose(rec[0, 0], want, rtol=1e-13, atol=1e-15)


def test_gamma_one_is_the_normalised_forms_numerator():
    """gamma = 1: the retention state is the running state S of the (separately pinned)
    normalised recurrence, and the last output is phi(q_N)^T S_N, its numerator."""
    Q, K, V = _rand(13, 2, 2, 30, 6, 5)
    _, Sr = oracle.retention_recurrent("elu1", Q, K, V, 1.0)
    Oret, _ = oracle.retention_recurrent("elu1", Q, K, V, 1.0)
    _, Sn, _ = oracle.causal_recurrent("elu1", Q, K, V)
    np.testing.assert_allclose(Sr, Sn, rtol=1e-13, atol=1e-13)
    for b in range(2):
        for h in range(2):
            num, _ = oracle.state_read(oracle.phi("elu1", Q[b, h, -1:]), Sn[b, h], np.ones(6))
            np.testing.assert_allclose(Oret[b, h, -1], num[0], rtol=1e-12, atol=1e-13)


def test_linear_in_values_and_state_handoff():
    Q, K, V = _rand(14, 1, 2, 25, 4, 3)
    V2 = np.random.default_rng(15).standard_normal(V.shape)
    g = [0.6, 0.99]
    a, _ = oracle.retention_recurrent("identity", Q, K, V, g)
    b, _ = oracle.retention_recurrent("identity", Q, K, V2, g)
    c, _ = oracle.retention_recurrent("identity", Q, K, 2.0 * V - 3.0 * V2, g)
    np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, rtol=1e-12, atol=1e-12)
    full, Sfull = oracle.retention_recurrent("identity", Q, K, V, g)
    for M in (1, 7, 24):
        o1, S1 = oracle.retention_recurrent("identity", Q[:, :, :M], K[:, :, :M], V[:, :, :M], g)
        o2, S2 = oracle.retention_chunked("identity", Q[:, :, M:], K[:, :, M:], V[:, :, M:], g, 4, S_in=S1)
        np.testing.assert_allclose(np.concatenate([o1, o2], 2), full, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S2, Sfull, rtol=1e-12, atol=1e-12)


def test_decode_steps_reproduce_forward():
    Q, K, V = _rand(16, 2, 2, 10, 4, 3)
    g = [0.5, 0.97]
    full, Sfull = oracle.retention_recurrent("identity", Q, K, V, g)
    S = np.zeros((2, 2, 4, 3))
    for i in range(10):
        o, S = oracle.retention_decode_step("identity", Q[:, :, i], K[:, :, i], V[:, :, i], S, g)
        np.testing.assert_allclose(o, full[:, :, i], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S, Sfull, rtol=1e-13, atol=1e-13)
