"""Pins of the oracle's state snapshots (CPU only).

Snapshot s of a sequence is the state before its token s * split_size.  It is
pinned against the brute-force product form (explicit prefix products of the
per-token transition matrices, no rank-1 update) run on the sequence's first
s * split_size tokens, for GDN and KDA, fixed-length and varlen."""

import numpy as np
import pytest

import oracle
from tests.test_oracle_recurrence import brute_force, rand_problem


def _prefix_state(q, k, v, beta, g, gk, h0, b, bos, t, n):
    """State of sequence n (batch row b, first token bos) before token t."""
    h0n = None if h0 is None else h0[n:n + 1]
    if t == bos:
        HV, V, K = v.shape[2], v.shape[3], q.shape[3]
        return np.zeros((HV, V, K)) if h0 is None else h0[n]
    sl = slice(bos, t)
    _, ht = brute_force(q[b:b + 1, sl], k[b:b + 1, sl], v[b:b + 1, sl], beta[b:b + 1, sl], 0.5,
                        g=None if g is None else g[b:b + 1, sl], gk=None if gk is None else gk[b:b + 1, sl],
                        h0=h0n)
    return ht[0]


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("S", [2, 3])
def test_snapshots_fixed_length(kda, S):
    rng = np.random.default_rng(10 + S + 2 * kda)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=7, Hk=1, HV=2, K=4, V=3, kda=kda)
    o, ht, hs = oracle.delta_rule_recurrent(q, k, v, beta, 0.5, g=g, gk=gk, h0=h0, split_size=S)
    per = -(-7 // S)
    assert hs.shape == (2 * per, 2, 3, 4)
    for b in range(2):
        for s in range(per):
            want = _prefix_state(q, k, v, beta, g, gk, h0, b, 0, s * S, b)
            np.testing.assert_allclose(hs[b * per + s], want, atol=1e-12)
    assert np.array_equal(hs[0], h0[0]) and np.array_equal(hs[per], h0[1])


def test_snapshots_varlen_offsets():
    rng = np.random.default_rng(20)
    lens = [5, 0, 3, 4]
    T = sum(lens)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=T, Hk=1, HV=2, K=4, V=3)
    h0 = rng.standard_normal((len(lens), 2, 3, 4)) * 0.1
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = 2
    o, ht, hs = oracle.delta_rule_recurrent(q, k, v, beta, 0.5, g=g, h0=h0, cu_seqlens=cu, split_size=S)
    counts = [-(-L // S) for L in lens]
    assert hs.shape[0] == sum(counts)
    i = 0
    for n, L in enumerate(lens):
        for s in range(counts[n]):
            want = _prefix_state(q, k, v, beta, g, None, h0, 0, cu[n], cu[n] + s * S, n)
            np.testing.assert_allclose(hs[i], want, atol=1e-12)
            i += 1


def test_snapshot_mutants_are_caught():
    """Recording after the token's update, or at the wrong phase, fails the pin."""
    import inspect
    import types
    import oracle.recurrence as rec
    rng = np.random.default_rng(30)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=6, Hk=1, HV=1, K=3, V=3)
    for old, new in [("(t - bos) % split_size == 0", "(t - bos) % split_size == split_size - 1"),
                     ("                snap[hs] = S\n", "                snap[hs] = S * 0.5 + S * 0.5 * (t > bos)\n")]:
        src = inspect.getsource(rec)
        assert old in src
        m = types.ModuleType("rec_mutant")
        exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), m.__dict__)
        _, _, hs = m.delta_rule_recurrent(q, k, v, beta, 0.5, g=g, h0=h0, split_size=2)
        ok = all(np.allclose(hs[s], _prefix_state(q, k, v, beta, g, None, h0, 0, 0, 2 * s, 0), atol=1e-12)
                 for s in range(hs.shape[0]))
        assert not ok, new
