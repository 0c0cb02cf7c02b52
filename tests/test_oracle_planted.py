"""Planted mistakes: a mutated copy of the oracle must fail the pins.

Each case rewrites one expression of ``oracle/recurrence.py`` or
``oracle/intra.py`` (a dropped term, a flipped sign, a transposed operand, a
wrong index), executes the mutated source as a throw-away module on the CPU,
and checks that the brute-force / closed-form pins reject it.  This shows the
pins are strong enough to catch plausible slips.
"""

import inspect
import types

import numpy as np
import pytest

import oracle.recurrence as rec
import oracle.intra as intra
from tests.test_oracle_recurrence import brute_force, rand_problem
from tests.test_oracle_intra import loop_intra


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert old in src, old
    src = src.replace(old, new, 1)
    src = src.replace("from .recurrence import", "from oracle.recurrence import")
    m = types.ModuleType(module.__name__ + "_mutant")
    exec(compile(src, "<mutant>", "exec"), m.__dict__)
    return m


REC_MUTATIONS = [
    ("v[b, t, hs] - pred", "pred - v[b, t, hs]"),                          # sign of the delta
    ("S += delta[:, :, None] * kt[:, None, :]", "S += delta[:, None, :] * kt[:, :, None]"),  # transposed update
    ("np.exp(g[b, t, hs])", "np.exp(-g[b, t, hs])"),                       # gate sign
    ("np.exp(gk[b, t, hs])[:, None, :]", "np.exp(gk[b, t, hs])[:, :, None]"),  # KDA gate on the wrong axis
    ("beta[b, t, hs][:, None] * (", "("),                                  # dropped beta
    ('np.einsum("hvk,hk->hv", S, qt)', 'np.einsum("hvk,hk->hv", S, kt)'),   # output with k instead of q
    ("kh = hs // (HV // Hk)", "kh = hs % Hk"),                             # wrong GQA head map
]


@pytest.mark.parametrize("old,new", REC_MUTATIONS)
def test_recurrence_mutant_is_caught(old, new):
    m = _mutant(rec, old, new)
    rng = np.random.default_rng(0)
    kda = "gk" in old
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=6, Hk=2, HV=4, K=4, V=4, kda=kda)
    o, ht = m.delta_rule_recurrent(q, k, v, beta, 0.7, g=g, gk=gk, h0=h0)
    ob, hb = brute_force(q, k, v, beta, 0.7, g=g, gk=gk, h0=h0)
    assert not (np.allclose(o, ob, atol=1e-9) and np.allclose(ht, hb, atol=1e-9))


INTRA_MUTATIONS = [
    ("diff = G[:, None, :] - G[None, :, :]", "diff = G[None, :, :] - G[:, None, :]"),  # gate difference reversed
    ("A = beta[b, rows, j][:, None] *", "A = beta[b, rows, j][None, :] *"),           # beta on columns
    ("strict = np.tril(np.ones((n, n), dtype=bool), -1)", "strict = np.tril(np.ones((n, n), dtype=bool))"),  # diagonal kept
    ('"tc,sc,tsc->ts", qc, kc', '"tc,sc,tsc->ts", kc, qc'),                              # transposed Aqk
]


@pytest.mark.parametrize("old,new", INTRA_MUTATIONS)
def test_intra_mutant_is_caught(old, new):
    m = _mutant(intra, old, new)
    rng = np.random.default_rng(1)
    q, k, v, beta, g, gk, h0 = rand_problem(rng, B=1, T=9, Hk=1, HV=1, K=3, V=3, kda=True)
    Aqk, Ainv = m.chunk_intra_matrices(q, k, beta, 0.6, gk=gk, chunk_size=16)
    Aqk_l, Akk_l = loop_intra(q, k, beta, 0.6, gk, 16)
    X = np.linalg.inv(np.eye(9) + Akk_l[0, :, 0, :9])
    ok_q = np.allclose(Aqk, Aqk_l, atol=1e-10)
    ok_i = np.allclose(Ainv[0, :, 0, :9], X, atol=1e-10)
    assert not (ok_q and ok_i)


HANDOFF_MUTATIONS = [
    ("out[p] = round_to_bf16(ht[n])", "out[p] = np.floor(ht[n] * 128) / 128"),   # not the bf16 rounding
    ("out[p] = round_to_bf16(ht[n])", "out[n] = round_to_bf16(ht[n])"),          # slot index ignored
    ("if 0 <= p < P:", "if 0 <= p <= P - 2:"),                                   # last slot skipped
]


@pytest.mark.parametrize("old,new", HANDOFF_MUTATIONS)
def test_handoff_mutant_is_caught(old, new):
    import oracle.handoff as handoff
    from tests import test_oracle_handoff as pins
    src = inspect.getsource(handoff)
    assert old in src, old
    src = src.replace(old, new, 1).replace("from .bf16 import", "from oracle.bf16 import")
    src = src.replace("from .recurrence import", "from oracle.recurrence import")
    m = types.ModuleType("handoff_mutant")
    exec(compile(src, "<mutant>", "exec"), m.__dict__)
    real = pins.oracle.state_to_pool
    pins.oracle.state_to_pool = m.state_to_pool
    try:
        failed = 0
        for t in (pins.test_handoff_matches_torch_cast_and_index_copy,
                  pins.test_handoff_identity_and_skipped_slots,
                  pins.test_handoff_rounding_is_nearest_even_at_planted_ties):
            try:
                t()
            except AssertionError:
                failed += 1
        assert failed > 0, "the handoff pins accepted a planted mistake"
    finally:
        pins.oracle.state_to_pool = real
