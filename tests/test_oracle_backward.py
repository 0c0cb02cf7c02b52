"""Pins of the oracle's backward state-gradient scan (CPU only).

The gradient at a chunk boundary is, by definition, the derivative of the loss
sum_t <do_t, o_t> + <dht, h_T> with respect to the state at that boundary.  The
pin computes exactly that with torch.autograd in float64: the state at the
boundary is a leaf, the decay-only forward runs from there to the sequence end
(k, v random: they enter additively), and its gradient is compared with the
oracle's reverse scan.  Planted mistakes must fail the pin."""

import inspect
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as bwd


def _problem(rng, B, T, Hk, HV, K, V, gate):
    q = rng.standard_normal((B, T, Hk, K))
    do = rng.standard_normal((B, T, HV, V))
    g = gk = gamma = gv = None
    if gate in ("gdn", "gdn+gv"):
        g = -np.logaddexp(0, rng.standard_normal((B, T, HV))) * 0.3
    if gate in ("gv", "gdn+gv"):
        gv = -np.logaddexp(0, rng.standard_normal((B, T, HV, V))) * 0.3
    if gate == "kda":
        gk = -np.logaddexp(0, rng.standard_normal((B, T, HV, K))) * 0.3
    elif gate == "gamma":
        gamma = -np.abs(rng.standard_normal(HV)) * 0.2
    return q, do, g, gk, gamma, gv


def _autograd_grad(q, do, g, gk, gamma, dht, scale, b, bos, eos, start, j, kh, rng, gv=None):
    """d loss / d state after token start - 1 (the state before token `start`)."""
    V, K = do.shape[3], q.shape[3]
    S0 = torch.zeros((V, K), dtype=torch.float64, requires_grad=True)
    S = S0
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(start, eos):
        if g is not None:
            S = S * float(np.exp(g[b, t, j]))
        if gamma is not None:
            S = S * float(np.exp(gamma[j]))
        if gk is not None:
            S = S * torch.from_numpy(np.exp(gk[b, t, j]))[None, :]
        if gv is not None:
            S = S * torch.from_numpy(np.exp(gv[b, t, j]))[:, None]
        kv = torch.from_numpy(np.outer(rng.standard_normal(V), rng.standard_normal(K)))
        S = S + kv
        o = scale * (S @ torch.from_numpy(q[b, t, kh]))
        loss = loss + o @ torch.from_numpy(do[b, t, j])
    if dht is not None:
        loss = loss + (S * torch.from_numpy(dht)).sum()
    if not loss.requires_grad:        # no token after `start` and no dht: the gradient is 0
        return np.zeros((V, K))
    loss.backward()
    return S0.grad.numpy()


@pytest.mark.parametrize("gate", ["gdn", "kda", "gamma", "gv", "gdn+gv", None])
def test_state_grad_matches_autograd(gate):
    rng = np.random.default_rng(50)
    B, T, Hk, HV, K, V, C = 1, 11, 1, 2, 4, 3, 4
    lens = [7, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, do, g, gk, gamma, gv = _problem(rng, B, T, Hk, HV, K, V, gate)
    dht = rng.standard_normal((len(lens), HV, V, K))
    dh, dh0 = oracle.state_grad_scan(q, do, 0.7, g=g, g_gamma=gamma, gk=gk, gv=gv, dht=dht, cu_seqlens=cu,
                                     split_size=2 * C, chunk_size=C)
    i = 0
    for n, L in enumerate(lens):
        bos, eos = cu[n], cu[n + 1]
        for j in range(HV):
            got = _autograd_grad(q, do, g, gk, gamma, dht[n, j], 0.7, 0, bos, eos, bos, j, 0, rng, gv=gv)
            np.testing.assert_allclose(dh0[n, j], got, atol=1e-12)
        nsnap = -(-L // (2 * C))
        for s in range(nsnap):
            end = min(bos + (2 * s + 1) * C, eos)   # end of chunk 2 s
            for j in range(HV):
                got = _autograd_grad(q, do, g, gk, gamma, dht[n, j], 0.7, 0, bos, eos, end, j, 0, rng, gv=gv)
                np.testing.assert_allclose(dh[i + s, j], got, atol=1e-12)
        i += nsnap
    assert dh.shape[0] == i


MUTATIONS = [
    ("""                    D = D + scale * np.outer(dout[b, t, j], q[b, t, kh])
                    if g is not None:
                        D = D * np.exp(g[b, t, jg])""", """                    if g is not None:
                        D = D * np.exp(g[b, t, jg])
                    D = D + scale * np.outer(dout[b, t, j], q[b, t, kh])"""),   # decay before the output term
    ("D = D + scale * np.outer(dout[b, t, j], q[b, t, kh])", "D = D + np.outer(dout[b, t, j], q[b, t, kh])"),  # scale dropped
    ("seq_snaps[ic // r][j] = D", "seq_snaps[ic // r][j] = D * 0 + dh0[n, j]"),  # snapshot of the wrong state
    ("D = D * np.exp(gv[b, t, jg])[:, None]", "D = D * np.exp(gv[b, t, jg])[None, :]"),   # gv on the key axis
    ("jg = j // (HV // Hg)", "jg = j % Hg"),                                                # wrong gate-head map
]


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_state_grad_mutant_is_caught(old, new):
    src = inspect.getsource(bwd)
    assert old in src
    src = src.replace(old, new, 1).replace("from .recurrence import", "from oracle.recurrence import")
    m = types.ModuleType("bwd_mutant")
    exec(compile(src, "<mutant>", "exec"), m.__dict__)
    rng = np.random.default_rng(51)
    # K = V: a wrong axis still runs; HV = 4 query / output heads share the
    # gates of Hg = 2 heads (the page's grouped form), so a wrong map shows
    q, do, g, gk, gamma, gv = _problem(rng, 1, 6, 4, 4, 3, 3, "gdn+gv")
    g, gv = g[:, :, :2], gv[:, :, :2]
    eg, egv = np.repeat(g, 2, axis=2), np.repeat(gv, 2, axis=2)
    dh, dh0 = m.state_grad_scan(q, do, 0.7, g=g, gv=gv, split_size=2, chunk_size=2)
    ok = True
    for j in range(4):
        ok = ok and np.allclose(dh0[0, j], _autograd_grad(q, do, eg, None, None, None, 0.7, 0, 0, 6, 0, j, j, rng,
                                                          gv=egv), atol=1e-12)
        ok = ok and all(np.allclose(dh[s, j], _autograd_grad(q, do, eg, None, None, None, 0.7, 0, 0, 6,
                                                               min(2 * s + 2, 6), j, j, rng, gv=egv), atol=1e-12)
                        for s in range(3))
    assert not ok


@pytest.mark.parametrize("gate", ["gdn", "kda", "gamma", "gdn+gv"])
def test_state_grad_grouped_gate_heads(gate):
    """The page's grouped form of chunk_bwd_kernel_dh: HQ = 4 query / output
    heads (q and dO per query head, one gradient each) read the gates of
    head i_hq // NG, NG = 2.  Pinned by autograd with the gates repeated per
    query head."""
    rng = np.random.default_rng(52)
    B, T, HQ, NG, K, V, C = 1, 9, 4, 2, 4, 3, 4
    q, do, g, gk, gamma, gv = _problem(rng, B, T, HQ, HQ, K, V, gate)
    H = HQ // NG
    cut = lambda x, ax: None if x is None else np.take(x, range(H), axis=ax)
    g, gk, gv, gamma = cut(g, 2), cut(gk, 2), cut(gv, 2), cut(gamma, 0)
    rep = lambda x, ax: None if x is None else np.repeat(x, NG, axis=ax)
    eg, egk, egv, egam = rep(g, 2), rep(gk, 2), rep(gv, 2), rep(gamma, 0)
    dht = rng.standard_normal((1, HQ, V, K))
    dh, dh0 = oracle.state_grad_scan(q, do, 0.7, g=g, g_gamma=gamma, gk=gk, gv=gv, dht=dht,
                                     split_size=C, chunk_size=C)
    for j in range(HQ):
        np.testing.assert_allclose(dh0[0, j], _autograd_grad(q, do, eg, egk, egam, dht[0, j], 0.7, 0, 0, T, 0, j, j,
                                                             rng, gv=egv), atol=1e-12)
        for s in range(-(-T // C)):
            end = min((s + 1) * C, T)
            np.testing.assert_allclose(dh[s, j], _autograd_grad(q, do, eg, egk, egam, dht[0, j], 0.7, 0, 0, T, end,
                                                                j, j, rng, gv=egv), atol=1e-12)
