"""Pins of the oracle's forward state scan (CPU only).

* Closed form: the state after tokens bos .. tau - 1 of a sequence is
      E(bos, tau) o h0 + sum_{s < tau} E(s + 1, tau) o (v_s k_s^T),
  with E(a, tau)[i, c] = exp(sum_{r = a .. tau-1} (g_r + gv_r[i] + gk_r[c]))
  -- every token's gate multiplies the terms added before it -- computed here
  from cumulative sums of the log-gates, not by stepping the recurrence.
  It is checked at every stored snapshot and at the end, with all gate forms,
  ragged and empty sequences, GQA heads and an initial state.
* No gate: ht = h0 + V^T K, a plain matrix product.
* Planted mistakes in the oracle must fail these pins."""

import importlib
import inspect
import types

import numpy as np
import pytest

import oracle
ss = importlib.import_module("oracle.state_scan")   # the module (the package binds the name to the function)


def _gates(rng, B, T, HV, K, V, forms):
    g = gamma = gk = gv = None
    if "g" in forms:
        g = -np.logaddexp(0, rng.standard_normal((B, T, HV))) * 0.3
    if "gamma" in forms:
        gamma = -np.abs(rng.standard_normal(HV)) * 0.2
    if "gk" in forms:
        gk = -np.logaddexp(0, rng.standard_normal((B, T, HV, K))) * 0.3
    if "gv" in forms:
        gv = -np.logaddexp(0, rng.standard_normal((B, T, HV, V))) * 0.3
    return g, gamma, gk, gv


def _closed_form(k, v, g, gamma, gk, gv, h0, b, bos, tau, j, kh):
    """State of (sequence at bos, head j) after the tokens bos .. tau - 1."""
    V, K = v.shape[3], k.shape[3]
    lam = np.zeros((tau - bos, V, K))           # per-token log-decay of each state entry
    for i, t in enumerate(range(bos, tau)):
        if g is not None:
            lam[i] += g[b, t, j]
        if gamma is not None:
            lam[i] += gamma[j]
        if gk is not None:
            lam[i] += gk[b, t, j][None, :]
        if gv is not None:
            lam[i] += gv[b, t, j][:, None]
    tail = np.cumsum(lam[::-1], axis=0)[::-1]   # tail[i] = sum of lam[i:]
    total = tail[0] if tau > bos else np.zeros((V, K))
    S = np.exp(total) * h0
    for i, t in enumerate(range(bos, tau)):
        after = tail[i + 1] if i + 1 < tau - bos else np.zeros((V, K))
        S = S + np.exp(after) * np.outer(v[b, t, j], k[b, t, kh])
    return S


@pytest.mark.parametrize("forms", [(), ("g",), ("gamma",), ("gk",), ("gv",), ("g", "gv"),
                                   ("gamma", "gv"), ("g", "gk", "gv")])
def test_state_scan_closed_form(forms):
    rng = np.random.default_rng(60)
    Hk, HV, K, V, C = 1, 2, 4, 3, 4
    lens = [9, 0, 4, 13]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = rng.standard_normal((1, T, Hk, K))
    v = rng.standard_normal((1, T, HV, V))
    g, gamma, gk, gv = _gates(rng, 1, T, HV, K, V, forms)
    h0 = rng.standard_normal((len(lens), HV, V, K))
    h, ht = oracle.state_scan(k, v, g=g, g_gamma=gamma, gk=gk, gv=gv, h0=h0, cu_seqlens=cu,
                              split_size=2 * C, chunk_size=C)
    i = 0
    for n, L in enumerate(lens):
        bos, eos = int(cu[n]), int(cu[n + 1])
        for j in range(HV):
            np.testing.assert_allclose(ht[n, j], _closed_form(k, v, g, gamma, gk, gv, h0[n, j], 0, bos, eos, j, 0),
                                       rtol=1e-12, atol=1e-12)
        nsnap = -(-L // (2 * C))
        for s in range(nsnap):
            start = bos + 2 * s * C                 # start of chunk 2 s
            for j in range(HV):
                np.testing.assert_allclose(h[i + s, j],
                                           _closed_form(k, v, g, gamma, gk, gv, h0[n, j], 0, bos, start, j, 0),
                                           rtol=1e-12, atol=1e-12)
        i += nsnap
    assert h.shape[0] == i


def test_state_scan_no_gate_is_matrix_product():
    rng = np.random.default_rng(61)
    B, T, Hk, HV, K, V = 2, 23, 2, 4, 5, 6
    k = rng.standard_normal((B, T, Hk, K))
    v = rng.standard_normal((B, T, HV, V))
    h0 = rng.standard_normal((B, HV, V, K))
    _, ht = oracle.state_scan(k, v, h0=h0, chunk_size=8)
    for b in range(B):
        for j in range(HV):
            np.testing.assert_allclose(ht[b, j], h0[b, j] + v[b, :, j].T @ k[b, :, j // 2], rtol=1e-12, atol=1e-12)


MUTATIONS = [
    ("""                    if g is not None:
                        S = S * np.exp(g[b, t, jg])
                    if gk""", """                    if gk"""),                                       # scalar gate dropped
    ("S = S * np.exp(gv[b, t, jg])[:, None]", "S = S * np.exp(gv[b, t, jg])[None, :]"),         # gv on the key axis
    ("S = S + np.outer(v[b, t, j], k[b, t, kh])", "S = S + np.outer(v[b, t, j], k[b, t, kh]) * np.exp(g[b, t, jg])"),
    ("seq_snaps[ic // r][j] = S", "seq_snaps[ic // r][j] = S * np.exp(g[b, bos, j])"),         # wrong snapshot
]


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_state_scan_mutant_is_caught(old, new):
    src = inspect.getsource(ss)
    assert old in src
    src = src.replace(old, new, 1).replace("from .recurrence import", "from oracle.recurrence import")
    m = types.ModuleType("ss_mutant")
    exec(compile(src, "<mutant>", "exec"), m.__dict__)
    rng = np.random.default_rng(62)
    K = V = 3
    k = rng.standard_normal((1, 7, 1, K))
    v = rng.standard_normal((1, 7, 1, V))
    g, _, _, gv = _gates(rng, 1, 7, 1, K, V, ("g", "gv"))
    h0 = rng.standard_normal((1, 1, V, K))
    h, ht = m.state_scan(k, v, g=g, gv=gv, h0=h0, split_size=2, chunk_size=2)
    ok = np.allclose(ht[0, 0], _closed_form(k, v, g, None, None, gv, h0[0, 0], 0, 0, 7, 0, 0), atol=1e-12)
    ok = ok and all(np.allclose(h[s, 0], _closed_form(k, v, g, None, None, gv, h0[0, 0], 0, 0, 2 * s, 0, 0),
                                atol=1e-12) for s in range(4))
    assert not ok


def _grouped_problem(rng, forms):
    """Gates with fewer heads than v (Hg = 2 of HV = 4), k per v-head."""
    Hk, HV, Hg, K, V = 4, 4, 2, 4, 3
    lens = [9, 5]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = rng.standard_normal((1, T, Hk, K))
    v = rng.standard_normal((1, T, HV, V))
    g, gamma, gk, gv = _gates(rng, 1, T, Hg, K, V, forms)
    h0 = rng.standard_normal((len(lens), HV, V, K))
    return lens, cu, k, v, (g, gamma, gk, gv), h0, HV // Hg


def _expand(gates, r):
    """The same gates repeated per v-head (head j gets gate head j // r)."""
    g, gamma, gk, gv = gates
    rep = lambda x, ax: None if x is None else np.repeat(x, r, axis=ax)
    return rep(g, 2), rep(gamma, 0), rep(gk, 2), rep(gv, 2)


@pytest.mark.parametrize("forms", [("g",), ("gamma", "gv"), ("gk",)])
def test_state_scan_grouped_gate_heads(forms):
    """The page's grouped form: v-head j takes gate head j // (HV / Hg).
    Checked against the closed form with the gates repeated per head."""
    rng = np.random.default_rng(63)
    lens, cu, k, v, gates, h0, r = _grouped_problem(rng, forms)
    g, gamma, gk, gv = gates
    h, ht = oracle.state_scan(k, v, g=g, g_gamma=gamma, gk=gk, gv=gv, h0=h0, cu_seqlens=cu,
                              split_size=4, chunk_size=4)
    eg, egam, egk, egv = _expand(gates, r)
    i = 0
    for n, L in enumerate(lens):
        bos, eos = int(cu[n]), int(cu[n + 1])
        for j in range(4):
            np.testing.assert_allclose(ht[n, j], _closed_form(k, v, eg, egam, egk, egv, h0[n, j], 0, bos, eos, j, j),
                                       rtol=1e-12, atol=1e-12)
            for s in range(-(-L // 4)):
                np.testing.assert_allclose(h[i + s, j], _closed_form(k, v, eg, egam, egk, egv, h0[n, j], 0, bos,
                                                                     bos + 4 * s, j, j), rtol=1e-12, atol=1e-12)
        i += -(-L // 4)


def test_state_scan_grouped_gate_mutant_is_caught():
    """A wrong gate-head map (j % Hg instead of j // (HV / Hg)) fails the pin."""
    src = inspect.getsource(ss)
    old = "jg = j // (HV // Hg)"
    assert old in src
    src = src.replace(old, "jg = j % Hg", 1).replace("from .recurrence import", "from oracle.recurrence import")
    m = types.ModuleType("ss_mutant")
    exec(compile(src, "<mutant>", "exec"), m.__dict__)
    rng = np.random.default_rng(64)
    lens, cu, k, v, gates, h0, r = _grouped_problem(rng, ("g",))
    _, ht = m.state_scan(k, v, g=gates[0], h0=h0, cu_seqlens=cu, chunk_size=4)
    eg = _expand(gates, r)[0]
    assert not all(np.allclose(ht[0, j], _closed_form(k, v, eg, None, None, None, h0[0, j], 0, 0, 9, j, j),
                               atol=1e-12) for j in range(4))
