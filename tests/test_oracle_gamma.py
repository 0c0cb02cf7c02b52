"""Pins of the oracle's fixed per-head decay (g_gamma) form (CPU only)."""

import numpy as np

import oracle
from tests.test_oracle_recurrence import brute_force, rand_problem


def test_gamma_beta0_closed_form():
    """beta = 0: nothing is written, the state only decays, so
    o_t = scale * exp(gamma * (t - bos + 1)) * h0 q_t within each sequence."""
    rng = np.random.default_rng(40)
    lens = [5, 3]
    q, k, v, beta, g, gk, _ = rand_problem(rng, B=1, T=8, Hk=1, HV=2, K=4, V=3)
    beta = np.zeros_like(beta)
    h0 = rng.standard_normal((2, 2, 3, 4))
    gamma = np.array([-0.3, -0.05])
    cu = np.array([0, 5, 8])
    o, ht = oracle.gdn_recurrent(q, k, v, None, beta, 0.7, h0=h0, cu_seqlens=cu, g_gamma=gamma)
    for n, (bos, eos) in enumerate(zip(cu[:-1], cu[1:])):
        for t in range(bos, eos):
            for j in range(2):
                want = 0.7 * np.exp(gamma[j] * (t - bos + 1)) * h0[n, j] @ q[0, t, 0]
                np.testing.assert_allclose(o[0, t, j], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ht[n], np.exp(gamma[:, None, None] * (eos - bos)) * h0[n], rtol=1e-12)


def test_gamma_matches_brute_force():
    rng = np.random.default_rng(41)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=6, Hk=1, HV=2, K=4, V=3)
    gamma = np.array([-0.2, -0.7])
    o, ht = oracle.gdn_recurrent(q, k, v, None, beta, 0.5, h0=h0, g_gamma=gamma)
    ob, hb = brute_force(q, k, v, beta, 0.5, g=np.broadcast_to(gamma, (2, 6, 2)).copy(), h0=h0)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(ht, hb, atol=1e-12)
