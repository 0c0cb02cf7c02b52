"""Pins for the per-chunk intra matrices (Aqk, (I + Akk)^-1) of the oracle."""

import numpy as np
import pytest
import scipy.linalg

import oracle
from tests.chunked_ref import chunked_delta_rule
from tests.test_oracle_recurrence import rand_problem


def loop_intra(q, k, beta, scale, gk, BT):
    """Pure-Python double loop over (t, s, c); the gate factor of entry (t, s)
    is the product of the per-token decays exp(gk_u) for s < u <= t (no
    cumulative sums)."""
    B, T, Hk, K = q.shape
    HV = beta.shape[2]
    Aqk = np.zeros((B, T, HV, BT))
    Akk = np.zeros((B, T, HV, BT))
    for b in range(B):
        for j in range(HV):
            jk = j // (HV // Hk)
            for t in range(T):
                c0 = (t // BT) * BT
                for s in range(c0, t + 1):
                    accq = acck = 0.0
                    for c in range(K):
                        f = 1.0
                        for u in range(s + 1, t + 1):
                            f *= np.exp(gk[b, u, j, c])
                        accq += q[b, t, jk, c] * k[b, s, jk, c] * f
                        acck += k[b, t, jk, c] * k[b, s, jk, c] * f
                    Aqk[b, t, j, s - c0] = scale * accq
                    if s < t:
                        Akk[b, t, j, s - c0] = beta[b, t, j] * acck
    return Aqk, Akk


@pytest.mark.parametrize("T,BT", [(11, 4), (9, 16)])
def test_intra_matches_loop_definition(T, BT):
    rng = np.random.default_rng(T)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=T, Hk=1, HV=2, K=3, V=2, kda=True)
    Aqk, Ainv = oracle.chunk_intra_matrices(q, k, beta, 0.6, gk=gk, chunk_size=BT)
    Aqk_l, Akk_l = loop_intra(q, k, beta, 0.6, gk, BT)
    np.testing.assert_allclose(Aqk, Aqk_l, rtol=1e-12, atol=1e-14)
    # (I + Akk) Akk_inv = I on every chunk block, from the loop-built Akk
    B, HV = 2, 2
    for b in range(B):
        for j in range(HV):
            for c0 in range(0, T, BT):
                n = min(BT, T - c0)
                L = np.eye(n) + Akk_l[b, c0:c0 + n, j, :n]
                X = Ainv[b, c0:c0 + n, j, :n]
                np.testing.assert_allclose(L @ X, np.eye(n), rtol=0, atol=1e-12)
                # unit lower triangular, zeros beyond the chunk
                np.testing.assert_allclose(np.triu(X, 1), 0, atol=0)
                np.testing.assert_allclose(np.diag(X), 1, atol=1e-15)
                assert np.all(Ainv[b, c0:c0 + n, j, n:] == 0)
                assert np.all(Aqk[b, c0:c0 + n, j, n:] == 0)


def test_inverse_matches_triangular_solver():
    rng = np.random.default_rng(21)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=64, Hk=1, HV=1, K=16, V=4, kda=True)
    Aqk, Ainv = oracle.chunk_intra_matrices(q, k, beta, 1.0, gk=gk, chunk_size=64)
    # (I + Akk) built from the definition, inverted with a triangular solver
    G = np.cumsum(gk[0, :, 0], axis=0)
    kk = k[0, :, 0]
    A = np.zeros((64, 64))
    for t in range(64):
        for s in range(t):
            A[t, s] = beta[0, t, 0] * np.sum(kk[t] * kk[s] * np.exp(G[t] - G[s]))
    X = scipy.linalg.solve_triangular(np.eye(64) + A, np.eye(64), lower=True, unit_diagonal=True)
    np.testing.assert_allclose(Ainv[0, :, 0], X, rtol=1e-11, atol=1e-12)


def test_block_merge_identities():
    """The 16 x 16 block formulas of the pages' merge step hold for the
    oracle's inverse: X10 = -X11 A10 X00, X20 = -X22 (A20 X00 + A21 X10),
    X30 = -X33 (A30 X00 + A31 X10 + A32 X20), and the diagonal blocks are the
    inverses of (I + A_ii)."""
    rng = np.random.default_rng(22)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=64, Hk=1, HV=1, K=32, V=4, kda=False)
    _, X = oracle.chunk_intra_matrices(q, k, beta, 1.0, g=g, chunk_size=64)
    X = X[0, :, 0]
    G = np.cumsum(g[0, :, 0])
    kk = k[0, :, 0]
    A = np.tril(beta[0, :, 0][:, None] * (kk @ kk.T) * np.exp(G[:, None] - G[None, :]), -1)
    blk = lambda M, i, j: M[16 * i:16 * i + 16, 16 * j:16 * j + 16]
    I16 = np.eye(16)
    for i in range(4):
        np.testing.assert_allclose(blk(X, i, i) @ (I16 + blk(A, i, i)), I16, atol=1e-12)
    np.testing.assert_allclose(blk(X, 1, 0), -blk(X, 1, 1) @ blk(A, 1, 0) @ blk(X, 0, 0), atol=1e-12)
    np.testing.assert_allclose(blk(X, 2, 1), -blk(X, 2, 2) @ blk(A, 2, 1) @ blk(X, 1, 1), atol=1e-12)
    np.testing.assert_allclose(blk(X, 3, 2), -blk(X, 3, 3) @ blk(A, 3, 2) @ blk(X, 2, 2), atol=1e-12)
    np.testing.assert_allclose(
        blk(X, 2, 0), -blk(X, 2, 2) @ (blk(A, 2, 0) @ blk(X, 0, 0) + blk(A, 2, 1) @ blk(X, 1, 0)), atol=1e-12)
    np.testing.assert_allclose(
        blk(X, 3, 1), -blk(X, 3, 3) @ (blk(A, 3, 1) @ blk(X, 1, 1) + blk(A, 3, 2) @ blk(X, 2, 1)), atol=1e-12)
    np.testing.assert_allclose(
        blk(X, 3, 0), -blk(X, 3, 3) @ (blk(A, 3, 0) @ blk(X, 0, 0) + blk(A, 3, 1) @ blk(X, 1, 0)
                                       + blk(A, 3, 2) @ blk(X, 2, 0)), atol=1e-12)


@pytest.mark.parametrize("kda", [False, True])
def test_intra_matrices_reproduce_recurrence(kda):
    """Using the oracle's Aqk and Akk_inv inside the chunked form (intra term
    Aqk D plus inter term) reproduces the token-by-token recurrence, which is
    itself pinned by brute force.  Includes a ragged tail and varlen."""
    rng = np.random.default_rng(23 + kda)
    lens = [70, 9, 64, 130]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, beta, g, gk, _ = rand_problem(rng, B=1, T=T, Hk=1, HV=2, K=8, V=5, kda=kda)
    h0 = rng.standard_normal((len(lens), 2, 5, 8)) * 0.3
    intra = oracle.chunk_intra_matrices(q, k, beta, 0.45, g=g, gk=gk, cu_seqlens=cu, chunk_size=64)
    oc, hc = chunked_delta_rule(q, k, v, beta, 0.45, g=g, gk=gk, h0=h0, chunk=64,
                                cu_seqlens=cu, intra=intra)
    o, ht = oracle.delta_rule_recurrent(q, k, v, beta, 0.45, g=g, gk=gk, h0=h0, cu_seqlens=cu)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(hc, ht, rtol=1e-10, atol=1e-11)


def test_chunk_subset_matches_full():
    rng = np.random.default_rng(24)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=40, Hk=1, HV=2, K=4, V=2, kda=True)
    full = oracle.chunk_intra_matrices(q, k, beta, 1.0, gk=gk, chunk_size=16)
    part = oracle.chunk_intra_matrices(q, k, beta, 1.0, gk=gk, chunk_size=16, chunks=[1, 4], heads=[1])
    # chunk 1 = batch 0 tokens 16..31, chunk 4 = batch 1 tokens 16..31
    for b in range(2):
        for x, y in zip(full, part):
            np.testing.assert_allclose(y[b, 16:32, 1], x[b, 16:32, 1], rtol=0, atol=0)
            assert np.all(y[b, :16] == 0) and np.all(y[b, 32:] == 0)
