"""Pins of the oracle's backward pass (gradients of the causal form).

The pages give no gradients, so the backward is pinned to things that do not
come from its own code:
  * central finite differences of the oracle's forward (itself pinned to the
    pages) for every input element, with and without a starting state and a
    loss on the final state;
  * closed forms: one token (o_1 = v_1 whatever q and k are), and a starting
    state that enters the loss only through the final state;
  * invariances of the normalised form: o_i does not change when phi(q_i) is
    scaled (so phi(q_i) . dphi(q_i) = 0), nor when every phi(k_j) is scaled
    together (no starting state), and o_i moves by u when u is added to every
    v_j (so the dV rows sum to the dO rows).
A dropped term (g or h), a sign slip in h, a transposed state, an exclusive
instead of an inclusive reverse sum, or a wrong Jacobian of the map fails at
least one of them.
"""
import numpy as np
import pytest

import oracle
from kernelized_linear_attention_la_amd import inputs


def _loss(phi, Q, K, V, W, S_in, z_in, dO, dS_out, dz_out):
    O, S, z = oracle.causal_recurrent(phi, Q, K, V, W=W, S_in=S_in, z_in=z_in)
    L = float((O * dO).sum())
    if dS_out is not None:
        L += float((S * dS_out).sum()) + float((z * dz_out).sum())
    return L


def _fd(f, x, eps):
    """Central differences of the scalar f with respect to every element of x."""
    g = np.empty_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + eps
        up = f()
        flat[i] = keep - eps
        dn = f()
        flat[i] = keep
        gf[i] = (up - dn) / (2 * eps)
    return g


def _case(phi, seed, B=1, H=2, N=6, dk=3, dv=4, m=5, state=True, away=1e-2):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, N, dk)) * 0.7
    K = rng.standard_normal((B, H, N, dk)) * 0.7
    # keep ELU+1 inputs away from its kink at 0, where one-sided slopes differ
    Q[np.abs(Q) < away] = away
    K[np.abs(K) < away] = away
    V = rng.standard_normal((B, H, N, dv))
    W = inputs.iid_gaussian_rows(seed, m, dk) if phi == "favor" else None
    dp = m if phi == "favor" else dk
    S_in = z_in = dS_out = dz_out = None
    if state:
        # a positive starting state (as a prefix of positive features would leave)
        S_in = rng.standard_normal((B, H, dp, dv)) * 0.3
        z_in = rng.uniform(0.5, 2.0, (B, H, dp))
        dS_out = rng.standard_normal((B, H, dp, dv))
        dz_out = rng.standard_normal((B, H, dp))
    dO = rng.standard_normal((B, H, N, dv))
    return Q, K, V, W, S_in, z_in, dO, dS_out, dz_out


@pytest.mark.parametrize("phi", ["elu1", "favor"])
@pytest.mark.parametrize("state", [False, True])
def test_backward_matches_finite_differences(phi, state):
    Q, K, V, W, S_in, z_in, dO, dS_out, dz_out = _case(phi, 11 + state, state=state)
    dQ, dK, dV, dS_in, dz_in = oracle.causal_backward(phi, Q, K, V, dO, W=W, S_in=S_in, z_in=z_in,
                                                      dS_out=dS_out, dz_out=dz_out)
    f = lambda: _loss(phi, Q, K, V, W, S_in, z_in, dO, dS_out, dz_out)  # noqa: E731
    eps = 1e-6
    for x, g in ((Q, dQ), (K, dK), (V, dV)) + (((S_in, dS_in), (z_in, dz_in)) if state else ()):
        fd = _fd(f, x, eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7 * max(1.0, np.abs(fd).max()))


def test_backward_worked_example_matrices_match_finite_differences():
    # the n = 4, d = 4 matrices of the printed worked example (all entries >= 0)
    # with keys and queries nudged off the ELU kink at 0
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "t1_kernel_la_worked_example.json")))
    Q = np.array(g["Q"], float)[None, None] + 0.05
    K = np.array(g["K"], float)[None, None] + 0.05
    V = np.array(g["V"], float)[None, None]
    dO = np.arange(16, dtype=float).reshape(1, 1, 4, 4) / 7 - 1
    dQ, dK, dV, _, _ = oracle.causal_backward("elu1", Q, K, V, dO)
    f = lambda: _loss("elu1", Q, K, V, None, None, None, dO, None, None)  # noqa: E731
    for x, gr in ((Q, dQ), (K, dK), (V, dV)):
        np.testing.assert_allclose(gr, _fd(f, x, 1e-6), rtol=1e-6, atol=1e-8)


def test_single_token_closed_form():
    # o_1 = (phi(q).phi(k)) v / (phi(q).phi(k)) = v: only V has a gradient
    rng = np.random.default_rng(3)
    Q, K, V, dO = (rng.standard_normal((2, 3, 1, d)) for d in (5, 5, 4, 4))
    for phi, W in (("elu1", None), ("favor", inputs.iid_gaussian_rows(3, 8, 5))):
        dQ, dK, dV, dS_in, dz_in = oracle.causal_backward(phi, Q, K, V, dO, W=W)
        np.testing.assert_allclose(dQ, 0, atol=1e-13)
        np.testing.assert_allclose(dK, 0, atol=1e-13)
        np.testing.assert_allclose(dV, dO, rtol=1e-14, atol=1e-14)


def test_gradient_of_starting_state_through_final_state_only():
    # with dO = 0 the loss is <dS_out, S_in + ...> + <dz_out, z_in + ...>:
    # dS_in = dS_out, dz_in = dz_out exactly, and dV_j = dS_out^T phi(k_j)
    Q, K, V, W, S_in, z_in, dO, dS_out, dz_out = _case("elu1", 5, state=True)
    dO[:] = 0
    dQ, dK, dV, dS_in, dz_in = oracle.causal_backward("elu1", Q, K, V, dO, S_in=S_in, z_in=z_in,
                                                      dS_out=dS_out, dz_out=dz_out)
    np.testing.assert_array_equal(dS_in, dS_out)
    np.testing.assert_array_equal(dz_in, dz_out)
    np.testing.assert_allclose(dQ, 0, atol=0)
    phik = np.stack([oracle.phi("elu1", K[0, h]) for h in range(K.shape[1])])[None]
    np.testing.assert_allclose(dV, np.einsum("bhjf,bhfc->bhjc", phik, dS_out), rtol=1e-13, atol=1e-13)


def test_invariances_of_the_normalised_form():
    # positive inputs: phi(x) = x + 1 and its Jacobian is the identity, so dphi = dx
    rng = np.random.default_rng(9)
    B, H, N, d = 2, 2, 9, 4
    Q = rng.uniform(0.1, 1.5, (B, H, N, d))
    K = rng.uniform(0.1, 1.5, (B, H, N, d))
    V = rng.standard_normal((B, H, N, d))
    dO = rng.standard_normal((B, H, N, d))
    dQ, dK, dV, _, _ = oracle.causal_backward("elu1", Q, K, V, dO)
    # scale invariance in phi(q_i), row by row
    np.testing.assert_allclose(((Q + 1) * dQ).sum(-1), 0, atol=1e-12)
    # joint scale invariance in all phi(k_j) (no starting state)
    np.testing.assert_allclose(((K + 1) * dK).sum((-1, -2)), 0, atol=1e-12)
    # translation: adding u to every v_j adds u to every o_i
    np.testing.assert_allclose(dV.sum(2), dO.sum(2), rtol=1e-12, atol=1e-12)
