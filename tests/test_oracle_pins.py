"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle to something independent of it: a value
printed on the pages (tests/golden, with the citation inside each file), a
closed form, a library routine, an invariant the pages state, or agreement of
two forms of the oracle that share no loop (the explicit pairwise form and the
running-sum recurrence).  A plausible slip in the oracle (a transposed operand,
a dropped normaliser term, an exclusive instead of inclusive causal mask, a
read before the update, a state not carried across chunks, a wrong FAVOR+
factor) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from kernelized_linear_attention_la_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _t1():
    g = _golden("t1_kernel_la_worked_example.json")
    Q = np.array(g["Q"], float)[None, None]
    K = np.array(g["K"], float)[None, None]
    V = np.array(g["V"], float)[None, None]
    return g, Q, K, V


# --------------------------------------------------------------------------
# printed worked examples
# --------------------------------------------------------------------------
def test_t1_state_equals_printed_phiK_T_V():
    g, Q, K, V = _t1()
    printed = np.array(g["phiK_T_V"], float)
    _, S_nc, z_nc = oracle.noncausal("elu1", Q, K, V)
    np.testing.assert_array_equal(S_nc[0, 0], printed)
    # the causal running sum reaches the same matrix after the last token
    _, S_c, z_c = oracle.causal_recurrent("elu1", Q, K, V)
    np.testing.assert_array_equal(S_c[0, 0], printed)
    _, S_ch, _ = oracle.causal_chunked("elu1", Q, K, V, chunk=3)
    np.testing.assert_array_equal(S_ch[0, 0], printed)
    # z = phi(K)^T 1 = column sums of K + 1
    np.testing.assert_array_equal(z_nc[0, 0], (np.array(g["K"], float) + 1).sum(0))


def test_t1_row1_numerator_denominator_and_output():
    g, Q, K, V = _t1()
    O, S, z = oracle.noncausal("elu1", Q, K, V)
    phiq = oracle.phi("elu1", Q[0, 0])
    np.testing.assert_array_equal(phiq[0], np.array(g["phi_q1"], float))
    num, den = oracle.state_read(phiq[:1], S[0, 0], z[0, 0])
    np.testing.assert_array_equal(num[0], np.array(g["num_1"], float))
    assert den[0] == g["denom_1"]
    np.testing.assert_array_equal(np.round(O[0, 0, 0], g["output_decimals"]),
                                  np.array(g["output_1_2dp"]))


def test_t3_infini_memory_read():
    g = _golden("t3_infini_memory_read.json")
    Q = np.array(g["Q"], float)
    sq = oracle.phi("elu1", Q)
    np.testing.assert_array_equal(sq, np.array(g["sigma_Q"], float))
    num, den = oracle.state_read(sq, np.array(g["M"], float), np.array(g["z"], float))
    np.testing.assert_array_equal(num, np.array(g["numerator"], float))
    np.testing.assert_array_equal(den, np.array(g["denominator"], float))
    A = num / den[:, None]
    np.testing.assert_array_equal(np.round(A, g["A_global_decimals"]),
                                  np.array(g["A_global_printed"]))


def test_t1_causal_special_rows():
    """Row 1 of the causal output is v_1; the last row equals the non-causal last row."""
    g, Q, K, V = _t1()
    Oc, _, _ = oracle.causal_recurrent("elu1", Q, K, V)
    On, _, _ = oracle.noncausal("elu1", Q, K, V)
    np.testing.assert_array_equal(Oc[0, 0, 0], V[0, 0, 0])
    np.testing.assert_allclose(Oc[0, 0, -1], On[0, 0, -1], rtol=1e-15)
    # rows 2..3 differ from the non-causal ones (the mask matters here)
    assert not np.allclose(Oc[0, 0, 1], On[0, 0, 1])


# --------------------------------------------------------------------------
# feature maps
# --------------------------------------------------------------------------
def test_elu1_matches_library_elu():
    x = np.concatenate([np.linspace(-30, 30, 601), [0.0, -0.0, 1e-300, -1e-300, 5e-8, -5e-8]])
    got = oracle.phi("elu1", x[:, None])[:, 0]
    ref = torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64), alpha=1.0).numpy() + 1.0
    # elu(x) + 1 evaluated in fp64 carries an absolute error of about one ulp of 1
    np.testing.assert_allclose(got, ref, rtol=2.3e-16, atol=2.3e-16)
    # on x <= 0 the map is exp(x) exactly (no cancellation in the oracle)
    neg = x <= 0
    np.testing.assert_allclose(got[neg], torch.exp(torch.tensor(x[neg], dtype=torch.float64)).numpy(),
                               rtol=2.3e-16, atol=0)
    assert np.all(got > 0)


def test_favor_closed_forms():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 6)) * 0.7
    # W = 0: every feature equals exp(-|x|^2/2)/sqrt(m)
    m = 9
    got = oracle.phi("favor", x, np.zeros((m, 6)))
    ref = np.exp(-0.5 * (x ** 2).sum(1))[:, None] / math.sqrt(m) * np.ones((1, m))
    np.testing.assert_allclose(got, ref, rtol=1e-15)
    # one feature: exp(w.x - |x|^2/2); the 1/sqrt(m) factor is 1
    w = rng.standard_normal((1, 6))
    got1 = oracle.phi("favor", x, w)[:, 0]
    np.testing.assert_allclose(got1, np.exp(x @ w[0] - 0.5 * (x ** 2).sum(1)), rtol=1e-14)
    # feature r depends on row r of W only (no transposed projection)
    W2 = rng.standard_normal((3, 6))
    got2 = oracle.phi("favor", x, W2)
    for r in range(3):
        np.testing.assert_allclose(got2[:, r] * math.sqrt(3),
                                   np.exp(x @ W2[r] - 0.5 * (x ** 2).sum(1)), rtol=1e-14)


@pytest.mark.parametrize("orthogonal", [False, True])
def test_favor_unbiased_for_softmax_kernel(orthogonal):
    """E_w[phi(q)^T phi(k)] = exp(q^T k) (Performer / FAVOR+, Story of Attention Part 5, 1b)."""
    d = 8
    rng = np.random.default_rng(11)
    q = rng.standard_normal(d) * 0.35
    k = rng.standard_normal(d) * 0.35
    if orthogonal:
        W = inputs.orthogonal_gaussian_rows(77, 64 * 2048, d).astype(np.float64)
    else:
        W = inputs.iid_gaussian_rows(77, 64 * 2048, d)
    m = W.shape[0]
    pq = oracle.phi("favor", q[None], W)[0]
    pk = oracle.phi("favor", k[None], W)[0]
    terms = m * pq * pk  # one unbiased estimate of exp(q.k) per feature
    # rows are independent across orthogonal blocks of d: use block means as samples
    blocks = terms.reshape(-1, d).mean(1)
    mean = blocks.mean()
    se = blocks.std(ddof=1) / math.sqrt(blocks.size)
    target = math.exp(q @ k)
    assert abs(mean - target) < 4 * se, (mean, target, se)
    # and the estimate is sharp enough to mean something
    assert se < 0.01 * target


def test_favor_attention_approaches_softmax_attention():
    """With many features, FAVOR+ attention approximates softmax(Q K^T) V."""
    rng = np.random.default_rng(3)
    N, d = 12, 4
    Q = rng.standard_normal((1, 1, N, d)) * 0.5
    K = rng.standard_normal((1, 1, N, d)) * 0.5
    V = rng.standard_normal((1, 1, N, d))
    # the estimate's relative standard error is about sqrt(e^{2|q+k|^2}/m) ~ 1% at m = 2^20
    W = inputs.orthogonal_gaussian_rows(91, 1 << 20, d).astype(np.float64)
    O, _, _ = oracle.noncausal("favor", Q, K, V, W)
    ref = torch.softmax(torch.tensor(Q[0, 0]) @ torch.tensor(K[0, 0]).T, dim=-1) @ torch.tensor(V[0, 0])
    err = np.abs(O[0, 0] - ref.numpy()).max()
    assert err < 0.03, err
    # and a transposed or dropped factor would not converge: a small m is clearly worse
    W_small = inputs.orthogonal_gaussian_rows(91, 1 << 8, d).astype(np.float64)
    O_s, _, _ = oracle.noncausal("favor", Q, K, V, W_small)
    assert np.abs(O_s[0, 0] - ref.numpy()).max() > err
    # causal: the i-th row approximates softmax over j <= i
    Oc, _, _ = oracle.causal_recurrent("favor", Q, K, V, W)
    s = torch.tensor(Q[0, 0]) @ torch.tensor(K[0, 0]).T
    s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    refc = torch.softmax(s, -1) @ torch.tensor(V[0, 0])
    assert np.abs(Oc[0, 0] - refc.numpy()).max() < 0.03


# --------------------------------------------------------------------------
# two modes, one function (brute force on tiny inputs)
# --------------------------------------------------------------------------
def _tiny(seed, N=13, dk=5, dv=3, phi="elu1", m=0, B=2, H=2):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, N, dk))
    K = rng.standard_normal((B, H, N, dk))
    V = rng.standard_normal((B, H, N, dv))
    W = rng.standard_normal((m, dk)) * 0.5 if phi == "favor" else None
    if phi == "favor":
        Q *= 0.5; K *= 0.5
    return Q, K, V, W


@pytest.mark.parametrize("phi,m", [("elu1", 0), ("favor", 7)])
@pytest.mark.parametrize("with_state", [False, True])
def test_recurrent_equals_pairwise(phi, m, with_state):
    Q, K, V, W = _tiny(1, phi=phi, m=m)
    dp = m if phi == "favor" else Q.shape[-1]
    S_in = z_in = None
    if with_state:
        # a valid state: the sums of some other phi(k) v^T
        Kp = np.random.default_rng(9).standard_normal((2, 2, 6, Q.shape[-1])) * (0.5 if phi == "favor" else 1)
        Vp = np.random.default_rng(10).standard_normal((2, 2, 6, V.shape[-1]))
        _, S_in, z_in = oracle.noncausal(phi, Kp, Kp, Vp, W)
        assert S_in.shape[-2] == dp
    O_r, S_r, z_r = oracle.causal_recurrent(phi, Q, K, V, W, S_in, z_in)
    O_q = oracle.quadratic(phi, Q, K, V, W, S_in, z_in, causal=True)
    np.testing.assert_allclose(O_r, O_q, rtol=1e-12, atol=1e-13)
    # the pairwise form with no mask equals the non-causal factorised form
    O_nc, S_nc, z_nc = oracle.noncausal(phi, Q, K, V, W)
    np.testing.assert_allclose(oracle.quadratic(phi, Q, K, V, W, causal=False), O_nc, rtol=1e-12, atol=1e-13)
    if not with_state:
        np.testing.assert_allclose(S_r, S_nc, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(z_r, z_nc, rtol=1e-12)


@pytest.mark.parametrize("phi,m", [("elu1", 0), ("favor", 6)])
def test_chunk_size_does_not_change_result(phi, m):
    N = 11
    Q, K, V, W = _tiny(2, N=N, phi=phi, m=m)
    O_r, S_r, z_r = oracle.causal_recurrent(phi, Q, K, V, W)
    for C in range(1, N + 2):
        O_c, S_c, z_c = oracle.causal_chunked(phi, Q, K, V, C, W)
        np.testing.assert_allclose(O_c, O_r, rtol=1e-12, atol=1e-13, err_msg=f"C={C}")
        np.testing.assert_allclose(S_c, S_r, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(z_c, z_r, rtol=1e-12)


def test_chunked_with_initial_state_matches_pairwise():
    Q, K, V, W = _tiny(4, N=10)
    rng = np.random.default_rng(8)
    S_in = rng.random((2, 2, 5, 3)) * 2
    z_in = rng.random((2, 2, 5)) + 0.5
    O_q = oracle.quadratic("elu1", Q, K, V, None, S_in, z_in, causal=True)
    for C in (1, 3, 4, 10, 16):
        O_c, _, _ = oracle.causal_chunked("elu1", Q, K, V, C, None, S_in, z_in)
        np.testing.assert_allclose(O_c, O_q, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# invariants of a normalised non-negative weighting
# --------------------------------------------------------------------------
def test_constant_values_and_convex_hull_and_linearity():
    Q, K, V, W = _tiny(5, N=17, dv=4)
    c = np.array([1.5, -2.0, 0.25, 7.0])
    Vc = np.broadcast_to(c, V.shape).copy()
    O, _, _ = oracle.causal_recurrent("elu1", Q, K, Vc)
    np.testing.assert_allclose(O, Vc, rtol=1e-13)
    O1, _, _ = oracle.causal_recurrent("elu1", Q, K, V)
    # row i lies inside the per-coordinate range of v_1..v_i
    lo = np.minimum.accumulate(V, axis=2)
    hi = np.maximum.accumulate(V, axis=2)
    assert np.all(O1 >= lo - 1e-12) and np.all(O1 <= hi + 1e-12)
    np.testing.assert_allclose(O1[:, :, 0], V[:, :, 0], rtol=1e-13)
    # linear in V
    V2 = np.random.default_rng(6).standard_normal(V.shape)
    O2, _, _ = oracle.causal_recurrent("elu1", Q, K, V2)
    O12, _, _ = oracle.causal_recurrent("elu1", Q, K, 2.0 * V - 3.0 * V2)
    np.testing.assert_allclose(O12, 2.0 * O1 - 3.0 * O2, rtol=1e-11, atol=1e-12)


def test_noncausal_key_permutation_invariance():
    Q, K, V, W = _tiny(6, N=9)
    perm = np.random.default_rng(1).permutation(9)
    O, S, z = oracle.noncausal("elu1", Q, K, V)
    Op, Sp, zp = oracle.noncausal("elu1", Q, K[:, :, perm], V[:, :, perm])
    np.testing.assert_allclose(Op, O, rtol=1e-12)
    np.testing.assert_allclose(Sp, S, rtol=1e-12)


# --------------------------------------------------------------------------
# decode = recurrence; state hand-off
# --------------------------------------------------------------------------
@pytest.mark.parametrize("phi,m", [("elu1", 0), ("favor", 5)])
def test_decode_steps_reproduce_forward(phi, m):
    Q, K, V, W = _tiny(7, N=8, phi=phi, m=m)
    dp = m if phi == "favor" else Q.shape[-1]
    O, S_f, z_f = oracle.causal_recurrent(phi, Q, K, V, W)
    S = np.zeros((2, 2, dp, V.shape[-1]))
    z = np.zeros((2, 2, dp))
    for t in range(Q.shape[2]):
        o, S, z = oracle.decode_step(phi, Q[:, :, t], K[:, :, t], V[:, :, t], S, z, W)
        np.testing.assert_allclose(o, O[:, :, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_f, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z, z_f, rtol=1e-12)


def test_state_handoff_split_anywhere():
    Q, K, V, W = _tiny(8, N=12)
    O, S, z = oracle.causal_recurrent("elu1", Q, K, V)
    for M in (1, 5, 7, 11):
        O1, S1, z1 = oracle.causal_chunked("elu1", Q[:, :, :M], K[:, :, :M], V[:, :, :M], 4)
        O2, S2, z2 = oracle.causal_chunked("elu1", Q[:, :, M:], K[:, :, M:], V[:, :, M:], 4, None, S1, z1)
        np.testing.assert_allclose(np.concatenate([O1, O2], 2), O, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(z2, z, rtol=1e-12)


# --------------------------------------------------------------------------
# input generator sanity (the values both sides receive)
# --------------------------------------------------------------------------
def test_generator_is_seeded_and_rounds_to_storage_format():
    a = inputs.custom_inputs(3, 1, 2, 5, 4, 4, dtype="bf16")
    b = inputs.custom_inputs(3, 1, 2, 5, 4, 4, dtype="bf16")
    np.testing.assert_array_equal(a.Q.store, b.Q.store)
    # every bf16 value survives a round trip through torch's bfloat16
    t = torch.tensor(a.K.f32).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(t, a.K.f32)
    assert a.K.store.dtype == np.uint16
    # slice (b, h) of a larger draw equals the same slice drawn alone
    big = inputs.normal_bhnd(9, 1, (2, 3, 4, 5), 0.5, "f32")
    one = inputs.normal_bhnd(9, 1, (2, 3, 4, 5), 0.5, "f32")
    np.testing.assert_array_equal(big.f32, one.f32)


def test_orthogonal_rows_are_orthogonal_within_blocks():
    W = inputs.orthogonal_gaussian_rows(5, 256, 64).astype(np.float64)
    for blk in range(4):
        Wb = W[blk * 64:(blk + 1) * 64]
        G = Wb @ Wb.T
        off = G - np.diag(np.diag(G))
        assert np.abs(off).max() < 1e-3 * np.diag(G).mean()
    # row lengths behave like |N(0, I_64)|: mean of |w|^2 close to 64
    assert abs((W ** 2).sum(1).mean() - 64) < 4 * math.sqrt(2 * 64 / 256) * 1.5


# --------------------------------------------------------------------------
# the normaliser near zero ("Story of Attention Part 5", 1a: phi(q)^T z can
# drift toward zero and make the division unstable).  Strongly negative ELU+1
# inputs put every feature on the exp branch, so phi(q).phi(k) is tiny.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("c", [-20.0, -60.0, -200.0])
def test_tiny_normaliser_constant_rows_give_running_mean(c):
    # every query and key row equal to the constant c < 0: all scores are the
    # same number exp(2c) d, so each causal output is the plain mean of the
    # values seen so far, and the non-causal output is the mean of all values
    rng = np.random.default_rng(11)
    B, H, N, dk, dv = 1, 2, 9, 4, 3
    Q = np.full((B, H, N, dk), c)
    K = np.full((B, H, N, dk), c)
    V = rng.standard_normal((B, H, N, dv))
    run_mean = np.cumsum(V, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    for O in (oracle.causal_recurrent("elu1", Q, K, V)[0], oracle.quadratic("elu1", Q, K, V),
              oracle.causal_chunked("elu1", Q, K, V, chunk=4)[0]):
        np.testing.assert_allclose(O, run_mean, rtol=1e-12, atol=1e-12)
    On = oracle.noncausal("elu1", Q, K, V)[0]
    np.testing.assert_allclose(On, np.broadcast_to(V.mean(axis=2, keepdims=True), On.shape), rtol=1e-12, atol=1e-12)
    # the normaliser itself is the count of tokens times exp(2c) d
    _, _, z = oracle.causal_recurrent("elu1", Q, K, V)
    np.testing.assert_allclose(z, N * math.exp(c), rtol=1e-12)


def test_tiny_normaliser_shift_invariance():
    # on the exp branch phi(x - s) = exp(-s) phi(x): shifting every coordinate
    # of all-negative query rows (or of all-negative keys, with no starting
    # state) scales numerator and denominator alike, so the outputs do not move
    rng = np.random.default_rng(12)
    B, H, N, dk, dv = 1, 2, 11, 5, 3
    Q = -np.abs(rng.standard_normal((B, H, N, dk))) - 0.1
    K = -np.abs(rng.standard_normal((B, H, N, dk))) - 0.1
    V = rng.standard_normal((B, H, N, dv))
    O0 = oracle.causal_recurrent("elu1", Q, K, V)[0]
    for s, t in ((30.0, 0.0), (0.0, 30.0), (25.0, 45.0)):
        O = oracle.causal_recurrent("elu1", Q - s, K - t, V)[0]
        np.testing.assert_allclose(O, O0, rtol=1e-9, atol=1e-12)
        On = oracle.noncausal("elu1", Q - s, K - t, V)[0]
        np.testing.assert_allclose(On, oracle.noncausal("elu1", Q, K, V)[0], rtol=1e-9, atol=1e-12)
