"""Pins for the token-by-token oracle (CPU only).

Each test checks the oracle against something other than itself: explicit
products of per-token transition matrices, an independently written chunked
form, closed forms of degenerate cases, a hand-computed scalar example, or a
structural invariant (GQA, varlen packing, state hand-off, KDA == GDN when the
per-channel gate is constant across channels).
"""

import json
import os

import numpy as np
import pytest

import oracle
from tests.chunked_ref import chunked_delta_rule

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_problem(rng, B=2, T=7, Hk=1, HV=2, K=5, V=4, kda=False, h0=True, norm=True, gscale=0.3):
    q = rng.standard_normal((B, T, Hk, K))
    k = rng.standard_normal((B, T, Hk, K))
    if norm:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, HV, V))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, HV))))
    g = gk = None
    if kda:
        gk = -np.logaddexp(0, rng.standard_normal((B, T, HV, K))) * gscale
    else:
        g = -np.logaddexp(0, rng.standard_normal((B, T, HV))) * gscale
    h = rng.standard_normal((B, HV, V, K)) * 0.5 if h0 else None
    return q, k, v, beta, g, gk, h


def brute_force(q, k, v, beta, scale, g=None, gk=None, h0=None):
    """S_t = S_0 prod_{u<=t} M_u + sum_{s<=t} beta_s v_s k_s^T prod_{s<u<=t} M_u with
    M_u = D_u (I - beta_u k_u k_u^T), D_u = exp(g_u) I or diag(exp(gk_u)).
    Every prefix product is formed explicitly; no rank-1 update is used."""
    B, T, Hk, K = q.shape
    HV, V = v.shape[2:]
    o = np.zeros((B, T, HV, V))
    ht = np.zeros((B, HV, V, K))
    for b in range(B):
        for j in range(HV):
            jk = j // (HV // Hk)
            S0 = np.zeros((V, K)) if h0 is None else h0[b, j]
            M = []
            for t in range(T):
                D = np.diag(np.exp(gk[b, t, j])) if gk is not None else np.exp(g[b, t, j]) * np.eye(K)
                kk = k[b, t, jk]
                M.append(D @ (np.eye(K) - beta[b, t, j] * np.outer(kk, kk)))
            for t in range(T):
                P = np.eye(K)
                for u in range(t + 1):
                    P = P @ M[u]
                S = S0 @ P
                for s in range(t + 1):
                    Ps = np.eye(K)
                    for u in range(s + 1, t + 1):
                        Ps = Ps @ M[u]
                    S = S + beta[b, s, j] * np.outer(v[b, s, j], k[b, s, jk]) @ Ps
                o[b, t, j] = scale * S @ q[b, t, jk]
                if t == T - 1:
                    ht[b, j] = S
    return o, ht


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_product_form(kda, seed):
    rng = np.random.default_rng(seed)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=7, Hk=1, HV=2, K=5, V=4, kda=kda)
    o, ht = oracle.delta_rule_recurrent(q, k, v, beta, 0.7, g=g, gk=gk, h0=h0)
    ob, hb = brute_force(q, k, v, beta, 0.7, g=g, gk=gk, h0=h0)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ht, hb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kda", [False, True])
def test_brute_force_unnormalised_keys(kda):
    # keys not normalised: the erase term beta k k^T then has a non-unit scale
    rng = np.random.default_rng(5)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=6, Hk=2, HV=2, K=3, V=3, kda=kda, norm=False)
    o, ht = oracle.delta_rule_recurrent(q, k, v, beta, 1.3, g=g, gk=gk, h0=h0)
    ob, hb = brute_force(q, k, v, beta, 1.3, g=g, gk=gk, h0=h0)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht, hb, rtol=1e-12, atol=1e-12)


def test_hand_computed_scalar():
    with open(os.path.join(HERE, "golden", "scalar_recurrence.json")) as f:
        d = json.load(f)
    T = len(d["g"])
    shp = (1, T, 1, 1)
    q = np.array(d["q"]).reshape(shp)
    k = np.array(d["k"]).reshape(shp)
    v = np.array(d["v"]).reshape(shp)
    beta = np.array(d["beta"]).reshape(1, T, 1)
    g = np.array(d["g"]).reshape(1, T, 1)
    o, ht = oracle.gdn_recurrent(q, k, v, g, beta, d["scale"])
    np.testing.assert_allclose(o.ravel(), d["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ht.ravel(), [d["ht"]], rtol=0, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("chunk,T", [(4, 13), (16, 37), (64, 130), (16, 16), (64, 5)])
def test_chunked_form_agrees(kda, chunk, T):
    rng = np.random.default_rng(chunk * 100 + T)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=T, Hk=1, HV=2, K=8, V=6, kda=kda)
    o, ht = oracle.delta_rule_recurrent(q, k, v, beta, 0.35, g=g, gk=gk, h0=h0)
    oc, hc = chunked_delta_rule(q, k, v, beta, 0.35, g=g, gk=gk, h0=h0, chunk=chunk)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(hc, ht, rtol=1e-10, atol=1e-11)


def test_beta_zero_gate_zero_is_frozen_state():
    rng = np.random.default_rng(3)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=9, Hk=2, HV=4, K=6, V=5)
    o, ht = oracle.gdn_recurrent(q, k, v, np.zeros_like(g), np.zeros_like(beta), 0.5, h0=h0)
    np.testing.assert_allclose(ht, h0, rtol=0, atol=0)
    for b in range(2):
        for t in range(9):
            for j in range(4):  # q/k head of v-head j is j // 2
                np.testing.assert_allclose(o[b, t, j], 0.5 * h0[b, j] @ q[b, t, j // 2],
                                           rtol=0, atol=1e-13)


def test_beta_zero_pure_decay():
    # beta = 0: nothing is written; o_t = scale * exp(Ghat_t) S0 q_t with the
    # cumulative gate from the sequence start.
    rng = np.random.default_rng(4)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=11, Hk=1, HV=3, K=4, V=3)
    o, ht = oracle.gdn_recurrent(q, k, v, g, np.zeros_like(beta), 2.0, h0=h0)
    Gh = np.cumsum(g[0], axis=0)  # [T, HV]
    for t in range(11):
        for j in range(3):
            np.testing.assert_allclose(o[0, t, j], 2.0 * np.exp(Gh[t, j]) * h0[0, j] @ q[0, t, 0],
                                       rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ht[0], np.exp(Gh[-1])[:, None, None] * h0[0], rtol=1e-13)


@pytest.mark.parametrize("gated", [False, True])
def test_orthogonal_keys_reduce_to_linear_attention(gated):
    # With mutually orthogonal unit keys and a zero start state the erase
    # term never sees earlier writes, so the output is causal (gated) linear
    # attention: o = scale * tril(Q K^T * Gamma) (beta * V).
    rng = np.random.default_rng(7)
    K = V = 8
    T = 8
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Qm.T.reshape(1, T, 1, K)  # rows of an orthogonal matrix
    q = rng.standard_normal((1, T, 1, K))
    v = rng.standard_normal((1, T, 1, V))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, T, 1))))
    g = -np.abs(rng.standard_normal((1, T, 1))) * 0.4 if gated else np.zeros((1, T, 1))
    o, _ = oracle.gdn_recurrent(q, k, v, g, beta, 0.9)
    Gh = np.cumsum(g[0, :, 0])
    Gamma = np.exp(Gh[:, None] - Gh[None, :])
    att = np.tril((q[0, :, 0] @ k[0, :, 0].T) * Gamma)
    ref = 0.9 * att @ (beta[0, :, 0:1] * v[0, :, 0])
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-12, atol=1e-12)


def test_kda_constant_channel_gate_equals_gdn():
    rng = np.random.default_rng(11)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=10, Hk=1, HV=2, K=6, V=5)
    gk = np.repeat(g[..., None], 6, axis=-1)
    o1, h1 = oracle.gdn_recurrent(q, k, v, g, beta, 0.4, h0=h0)
    o2, h2 = oracle.kda_recurrent(q, k, v, gk, beta, 0.4, h0=h0)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(h2, h1, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_gqa_equals_repeated_heads(kda):
    rng = np.random.default_rng(12)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=9, Hk=2, HV=6, K=4, V=3, kda=kda)
    o1, h1 = oracle.delta_rule_recurrent(q, k, v, beta, 0.6, g=g, gk=gk, h0=h0)
    qr, kr = np.repeat(q, 3, axis=2), np.repeat(k, 3, axis=2)
    o2, h2 = oracle.delta_rule_recurrent(qr, kr, v, beta, 0.6, g=g, gk=gk, h0=h0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=0)
    np.testing.assert_allclose(h1, h2, rtol=0, atol=0)


@pytest.mark.parametrize("kda", [False, True])
def test_varlen_equals_separate_runs(kda):
    rng = np.random.default_rng(13)
    lens = [5, 1, 9, 3]
    T = sum(lens)
    q, k, v, beta, g, gk, _ = rand_problem(rng, B=1, T=T, Hk=1, HV=2, K=4, V=3, kda=kda)
    h0 = rng.standard_normal((len(lens), 2, 3, 4))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, ht = oracle.delta_rule_recurrent(q, k, v, beta, 0.8, g=g, gk=gk, h0=h0, cu_seqlens=cu)
    for n in range(len(lens)):
        s = slice(cu[n], cu[n + 1])
        o1, h1 = oracle.delta_rule_recurrent(
            q[:, s], k[:, s], v[:, s], beta[:, s], 0.8,
            g=None if g is None else g[:, s], gk=None if gk is None else gk[:, s], h0=h0[n:n + 1])
        np.testing.assert_allclose(o[:, s], o1, rtol=0, atol=0)
        np.testing.assert_allclose(ht[n], h1[0], rtol=0, atol=0)


@pytest.mark.parametrize("kda", [False, True])
def test_state_handoff(kda):
    rng = np.random.default_rng(14)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=2, T=12, Hk=1, HV=2, K=4, V=4, kda=kda)
    o, ht = oracle.delta_rule_recurrent(q, k, v, beta, 1.0, g=g, gk=gk, h0=h0)
    sl = lambda x, s: None if x is None else x[:, s]
    a, b = slice(0, 5), slice(5, 12)
    o1, h1 = oracle.delta_rule_recurrent(q[:, a], k[:, a], v[:, a], beta[:, a], 1.0,
                                         g=sl(g, a), gk=sl(gk, a), h0=h0)
    o2, h2 = oracle.delta_rule_recurrent(q[:, b], k[:, b], v[:, b], beta[:, b], 1.0,
                                         g=sl(g, b), gk=sl(gk, b), h0=h1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(h2, ht, rtol=1e-14, atol=1e-14)


def test_scale_is_linear():
    rng = np.random.default_rng(15)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=6, Hk=1, HV=1, K=4, V=4)
    o1, h1 = oracle.gdn_recurrent(q, k, v, g, beta, 1.0, h0=h0)
    o2, h2 = oracle.gdn_recurrent(q, k, v, g, beta, 0.25, h0=h0)
    np.testing.assert_allclose(o2, 0.25 * o1, rtol=1e-14)
    np.testing.assert_allclose(h2, h1, rtol=0, atol=0)


def test_head_subset_matches_full_run():
    rng = np.random.default_rng(16)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=8, Hk=2, HV=4, K=4, V=4)
    o, ht = oracle.gdn_recurrent(q, k, v, g, beta, 0.5, h0=h0)
    o2, h2 = oracle.gdn_recurrent(q, k, v, g, beta, 0.5, h0=h0, heads=[1, 2])
    np.testing.assert_allclose(o2[:, :, [1, 2]], o[:, :, [1, 2]], rtol=0, atol=0)
    np.testing.assert_allclose(h2[:, [1, 2]], ht[:, [1, 2]], rtol=0, atol=0)
