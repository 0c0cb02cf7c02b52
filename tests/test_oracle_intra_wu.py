"""Pins for the oracle's scalar-gate intra-chunk step with w and u
(oracle.chunk_intra_wu).

The checks that do not go through the function's own formulas: chained over
the chunks of a sequence, the WY update h <- e^{G_last} h + (K o
e^{G_last - G})^T (u - w h) must reproduce the token-by-token recurrence's
final state (oracle.gdn_recurrent, itself pinned by brute-force products in
test_oracle_recurrence.py) exactly up to fp64 rounding, for ragged chunks, GQA
heads and a nonzero initial state; A must equal the inverse that
chunk_intra_matrices forms from its own per-channel definition; the page's
cumulative-gate convention must give the same result as per-token gates; and
planted mistakes (a dropped beta, a missing gate factor) must fail the state
check."""

import numpy as np
import pytest

import oracle
from tests.test_oracle_recurrence import rand_problem


def _chained_state(k, v, g, h0, A, w, u, BT, cu=None):
    """Final states [N, HV, V, K] from the WY chunk updates, h = S^T (K x V)."""
    B, T, Hk, K = k.shape
    HV = v.shape[2]
    seqs = [(b, 0, T) for b in range(B)] if cu is None else [(0, int(a), int(e)) for a, e in zip(cu[:-1], cu[1:])]
    out = []
    for n, (b, bos, eos) in enumerate(seqs):
        hs = []
        for j in range(HV):
            h = h0[n, j].T.copy()                                   # [K, V]
            for c0 in range(bos, eos, BT):
                rows = slice(c0, min(c0 + BT, eos))
                G = np.cumsum(g[b, rows, j])
                kt = k[b, rows, j // (HV // Hk)] * np.exp(G[-1] - G)[:, None]
                h = np.exp(G[-1]) * h + kt.T @ (u[b, rows, j] - w[b, rows, j] @ h)
            hs.append(h.T)
        out.append(np.stack(hs))
    return np.stack(out)


@pytest.mark.parametrize("T,BT,Hk,HV", [(7, 4, 1, 2), (13, 4, 2, 4), (20, 8, 1, 1)])
def test_wy_update_reproduces_recurrence(T, BT, Hk, HV):
    rng = np.random.default_rng(T + BT)
    q, k, v, beta, g, _, h0 = rand_problem(rng, B=2, T=T, Hk=Hk, HV=HV, K=5, V=3)
    A, w, u = oracle.chunk_intra_wu(k, v, beta, g=g, chunk_size=BT)
    _, ht = oracle.gdn_recurrent(q, k, v, g, beta, 1.0, h0=h0)
    got = _chained_state(k, v, g, h0, A, w, u, BT)
    np.testing.assert_allclose(got, ht, rtol=0, atol=1e-11)


def test_wy_update_varlen():
    rng = np.random.default_rng(3)
    lens = [5, 0, 9, 1]
    q, k, v, beta, g, _, _ = rand_problem(rng, B=1, T=sum(lens), Hk=1, HV=2, K=4, V=3, h0=False)
    cu = np.concatenate([[0], np.cumsum(lens)])
    h0 = rng.standard_normal((len(lens), 2, 3, 4)) * 0.5
    A, w, u = oracle.chunk_intra_wu(k, v, beta, g=g, cu_seqlens=cu, chunk_size=4)
    _, ht = oracle.gdn_recurrent(q, k, v, g, beta, 1.0, h0=h0, cu_seqlens=cu)
    got = _chained_state(k, v, g, h0, A, w, u, 4, cu=cu)
    np.testing.assert_allclose(got, ht, rtol=0, atol=1e-11)


def test_inverse_matches_intra_matrices():
    rng = np.random.default_rng(5)
    q, k, v, beta, g, _, _ = rand_problem(rng, B=2, T=11, Hk=1, HV=2, K=6, V=3)
    A, _, _ = oracle.chunk_intra_wu(k, v, beta, g=g, chunk_size=4)
    _, Ainv = oracle.chunk_intra_matrices(q, k, beta, 1.0, g=g, chunk_size=4)
    np.testing.assert_allclose(A, Ainv, rtol=0, atol=1e-13)


def test_cumulative_gate_convention():
    rng = np.random.default_rng(6)
    _, k, v, beta, g, _, _ = rand_problem(rng, B=1, T=10, Hk=1, HV=2, K=4, V=3)
    G = np.zeros_like(g)
    for c0 in range(0, 10, 4):                    # chunk-local cumulative sums
        G[:, c0:c0 + 4] = np.cumsum(g[:, c0:c0 + 4], axis=1)
    a = oracle.chunk_intra_wu(k, v, beta, g=g, chunk_size=4)
    b = oracle.chunk_intra_wu(k, v, beta, g=G, chunk_size=4, g_cumulative=True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mistake", ["w_without_beta", "w_without_gate", "u_without_beta"])
def test_planted_mistakes_fail(mistake):
    rng = np.random.default_rng(7)
    q, k, v, beta, g, _, h0 = rand_problem(rng, B=1, T=9, Hk=1, HV=1, K=4, V=3)
    A, w, u = oracle.chunk_intra_wu(k, v, beta, g=g, chunk_size=4)
    w2, u2 = w.copy(), u.copy()
    for c0 in range(0, 9, 4):
        rows = slice(c0, min(c0 + 4, 9))
        Ainv = A[0, rows, 0, : rows.stop - c0]
        G = np.cumsum(g[0, rows, 0])
        if mistake == "w_without_beta":
            w2[0, rows, 0] = Ainv @ (np.exp(G)[:, None] * k[0, rows, 0])
        elif mistake == "w_without_gate":
            w2[0, rows, 0] = Ainv @ (beta[0, rows, 0][:, None] * k[0, rows, 0])
        else:
            u2[0, rows, 0] = Ainv @ v[0, rows, 0]
    _, ht = oracle.gdn_recurrent(q, k, v, g, beta, 1.0, h0=h0)
    assert np.abs(_chained_state(k, v, g, h0, A, w, u, 4) - ht).max() < 1e-11
    assert np.abs(_chained_state(k, v, g, h0, A, w2, u2, 4) - ht).max() > 1e-3
