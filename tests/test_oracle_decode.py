"""Pins for the decode oracle and the bf16 rounding (CPU only)."""

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def test_gate_against_library_routines():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((50, 8)) * 6
    b = rng.standard_normal((50, 8)) * 4
    A_log = rng.standard_normal(8)
    dt = rng.standard_normal(8)
    alpha, beta = oracle.decode_gate(a, b, A_log, dt)
    x = a + dt
    # log(1 + e^x) via logaddexp; the oracle switches to x above 20, where the
    # two differ by less than e^-20
    sp = np.logaddexp(0.0, x)
    np.testing.assert_allclose(alpha, np.exp(-np.exp(A_log) * sp), rtol=1e-8)
    np.testing.assert_allclose(beta, scipy.special.expit(b), rtol=1e-14)


def test_gate_threshold_branch_and_softplus_beta():
    x = np.array([[-3.0, 0.0, 19.9, 20.0, 20.1, 45.0]])
    alpha, _ = oracle.decode_gate(x, np.zeros_like(x), np.zeros(6), np.zeros(6))
    g = np.log(alpha)
    sp = np.array([np.log1p(np.exp(-3.0)), np.log(2.0), np.log1p(np.exp(19.9)), np.log1p(np.exp(20.0)), 20.1, 45.0])
    np.testing.assert_allclose(-g, sp[None], rtol=1e-12)
    # softplus with beta_sp = 2: log(1 + e^{2x}) / 2 below threshold 20 (2x <= 20)
    alpha2, _ = oracle.decode_gate(x, np.zeros_like(x), np.zeros(6), np.zeros(6), softplus_beta=2.0)
    sp2 = np.where(2 * x <= 20, np.logaddexp(0, 2 * x) / 2, x)
    np.testing.assert_allclose(-np.log(alpha2), sp2, rtol=1e-12)


def test_normalize_against_linalg_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 4, 128))
    y = oracle.decode_normalize(x, eps=0.0, scale=0.5)
    np.testing.assert_allclose(y, 0.5 * x / np.linalg.norm(x, axis=-1, keepdims=True), rtol=1e-14)
    y2 = oracle.decode_normalize(x, eps=1e-6)
    np.testing.assert_allclose(y2, x / np.sqrt(np.linalg.norm(x, axis=-1, keepdims=True) ** 2 + 1e-6),
                               rtol=1e-14)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(10000) * 10.0 ** rng.integers(-30, 30, 10000),
        [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4e38, 1e-40, -1e-42],
        # exact ties in bf16: 1 + 2^-8 (tie, round to even = 1), 1 + 3*2^-8 (tie, round up)
        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)],
    ])
    ours = oracle.round_to_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(ours, ref)
    assert ours[-3] == 1.0 and ours[-2] == 1.0 + 2.0 ** -6
    assert np.isnan(oracle.round_to_bf16(np.array([np.nan]))[0])


def _decode_problem(rng, B=3, T=4, H=2, HV=4, K=8, V=6, pool=None):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, HV, V))
    a = rng.standard_normal((B, T, HV))
    b = rng.standard_normal((B, T, HV))
    A_log = rng.standard_normal(HV) * 0.5
    dt = rng.standard_normal(HV)
    P = B if pool is None else pool
    state = oracle.round_to_bf16(rng.standard_normal((P, HV, V, K)) * 0.3)
    return q, k, v, a, b, A_log, dt, state


@pytest.mark.parametrize("T", [1, 2, 4])
def test_decode_equals_recurrence_with_gate_and_norm(T):
    """Decode of T tokens equals the (brute-force pinned) recurrence run on the
    normalised q/k with g = log(alpha), h0 = state, then rounded to bf16."""
    rng = np.random.default_rng(10 + T)
    q, k, v, a, b, A_log, dt, state = _decode_problem(rng, T=T)
    o, ns = oracle.gdn_decode(q, k, v, a, b, A_log, dt, state, scale=0.3)
    alpha, beta = oracle.decode_gate(a, b, A_log, dt)
    qn = q / np.sqrt((q ** 2).sum(-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt((k ** 2).sum(-1, keepdims=True) + 1e-6)
    for bi in range(3):
        ob, hb = oracle.gdn_recurrent(qn[bi:bi + 1], kn[bi:bi + 1], v[bi:bi + 1], np.log(alpha[bi:bi + 1]),
                                      beta[bi:bi + 1], 0.3, h0=state[bi:bi + 1])
        np.testing.assert_allclose(o[bi], ob[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(ns[bi], oracle.round_to_bf16(hb[0]))


def test_decode_without_norm_and_default_scale():
    rng = np.random.default_rng(20)
    q, k, v, a, b, A_log, dt, state = _decode_problem(rng, T=2, K=16)
    o, ns = oracle.gdn_decode(q, k, v, a, b, A_log, dt, state, use_qk_l2norm=False)
    alpha, beta = oracle.decode_gate(a, b, A_log, dt)
    ob, hb = oracle.gdn_recurrent(q, k, v, np.log(alpha), beta, 16 ** -0.5, h0=state)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(ns, oracle.round_to_bf16(hb))


def test_decode_pool_indices():
    """A pool larger than the batch with permuted slots: each batch row reads
    and writes its own slot; untouched slots keep their bits."""
    rng = np.random.default_rng(30)
    q, k, v, a, b, A_log, dt, state = _decode_problem(rng, B=3, T=2, pool=7)
    idx = np.array([5, 0, 3])
    o, ns = oracle.gdn_decode(q, k, v, a, b, A_log, dt, state, indices=idx)
    o_id, ns_id = oracle.gdn_decode(q, k, v, a, b, A_log, dt, state[idx])
    np.testing.assert_array_equal(o, o_id)
    np.testing.assert_array_equal(ns[idx], ns_id)
    for p in (1, 2, 4, 6):
        np.testing.assert_array_equal(ns[p], state[p])


def test_decode_batch_subset():
    rng = np.random.default_rng(31)
    q, k, v, a, b, A_log, dt, state = _decode_problem(rng, B=4, T=1)
    o, ns = oracle.gdn_decode(q, k, v, a, b, A_log, dt, state)
    o2, ns2 = oracle.gdn_decode(q, k, v, a, b, A_log, dt, state, batches=[2])
    np.testing.assert_array_equal(o2[2], o[2])
    np.testing.assert_array_equal(ns2[2], ns[2])
    np.testing.assert_array_equal(ns2[0], state[0])
