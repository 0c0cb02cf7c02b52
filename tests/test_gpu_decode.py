"""GPU parity of the decode kernel against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_61_amd import binding, workloads
from tests.tolerance import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(inp, batches=None, use_norm=True, sp_beta=1.0, sp_thr=20.0):
    d = {n: getattr(inp, n) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")}
    g = {n: t.to(DEV) for n, t in d.items()}
    state = inp.state.to(DEV).clone()
    idx = None if inp.indices is None else inp.indices.to(DEV)
    o = binding.gdn_decode(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], state,
                           idx, scale=inp.scale, use_qk_l2norm=use_norm, softplus_beta=sp_beta,
                           softplus_threshold=sp_thr)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gdn_decode(inp.q, inp.k, inp.v, inp.a, inp.b, inp.A_log, inp.dt_bias,
                                     inp.state, indices=inp.indices, scale=inp.scale,
                                     softplus_beta=sp_beta, softplus_threshold=sp_thr,
                                     use_qk_l2norm=use_norm, batches=batches, round_state=False)
    return o.cpu(), state.cpu(), o_ref, s_ref


def _ulp_consistent(s_gpu, s_exact):
    """The GPU's bf16 state is within one bf16 ulp of the oracle's state
    rounded to bf16 (the two roundings may straddle a rounding boundary),
    up to a floor of 1e-4 RMS for entries near zero, where the fp32
    arithmetic error exceeds their tiny ulp."""
    r = oracle.round_to_bf16(s_exact)
    g = to64(s_gpu)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    floor = 1e-4 * np.sqrt(np.mean(r * r))
    assert np.all(np.abs(g - r) <= ulp + floor), "state differs from the rounded oracle state by more than one ulp"


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_small(T):
    print(f"decode small T={T}", flush=True)
    inp = workloads.make_decode(3, T, 2, 4, 128, 128, seed=50 + T)
    o, s, o_ref, s_ref = _run(inp)
    check("o", o, o_ref, torch.bfloat16)
    check("state", s, s_ref, torch.bfloat16)
    _ulp_consistent(s, s_ref)


@pytest.mark.parametrize("B,T", [(1, 1), (1, 4), (7, 1), (7, 3), (8, 2), (31, 4)])
def test_decode_split_grid_sizes(B, T):
    """Batches on both sides of the work-group split (fewer than 256
    (batch row, v-head) pairs run four 64-thread work-groups per pair), with
    the workload's head shape (16 q/k heads, 32 v-heads) and a pool larger
    than the batch with shuffled slots."""
    print(f"decode split-grid B={B} T={T}", flush=True)
    rng = np.random.default_rng(70 + B + T)
    pool = B + 3
    idx = rng.permutation(pool)[:B].tolist()
    inp = workloads.make_decode(B, T, 16, 32, 128, 128, seed=71 + B, pool=pool, indices=idx)
    o, s, o_ref, s_ref = _run(inp)
    check("o", o, o_ref, torch.bfloat16)
    used = np.zeros(pool, bool)
    used[idx] = True
    tused = torch.from_numpy(used)
    check("state", s[tused], s_ref[used], torch.bfloat16)
    assert torch.equal(s[~tused], inp.state[~tused]), "slots outside the batch changed"


def test_decode_no_norm():
    inp = workloads.make_decode(2, 2, 1, 2, 128, 128, seed=61)
    inp.q = (inp.q.float() * 0.1).to(torch.bfloat16)
    inp.k = (inp.k.float() * 0.1).to(torch.bfloat16)
    o, s, o_ref, s_ref = _run(inp, use_norm=False)
    check("o", o, o_ref, torch.bfloat16)
    check("state", s, s_ref, torch.bfloat16)


def test_decode_pool_indices_and_invalid_slot():
    print("decode pool", flush=True)
    inp = workloads.make_decode(4, 2, 2, 4, 128, 128, seed=62, pool=9, indices=[7, 0, 4, 2])
    o, s, o_ref, s_ref = _run(inp)
    check("o", o, o_ref, torch.bfloat16)
    check("state", s, s_ref, torch.bfloat16)
    untouched = [1, 3, 5, 6, 8]
    assert torch.equal(s[untouched], inp.state[untouched])
    # an out-of-range slot: o = 0, pool untouched
    bad = workloads.make_decode(2, 1, 2, 4, 128, 128, seed=63, pool=3, indices=[1, 3])
    state = bad.state.to(DEV).clone()
    o = binding.gdn_decode(bad.q.to(DEV), bad.k.to(DEV), bad.v.to(DEV), bad.a.to(DEV), bad.b.to(DEV),
                           bad.A_log.to(DEV), bad.dt_bias.to(DEV), state, bad.indices.to(DEV))
    torch.cuda.synchronize()
    assert torch.all(o[1].float() == 0)
    st = state.cpu()
    assert torch.equal(st[0], bad.state[0]) and torch.equal(st[2], bad.state[2])
    assert not torch.equal(st[1], bad.state[1])


@pytest.mark.parametrize("T", [1, 4])
def test_decode_b256_sampled(T):
    """The full B=256, HV=32 workload; the oracle checks 12 sampled rows."""
    print(f"decode B256 T={T}", flush=True)
    inp = workloads.decode_b256(T)
    rows = sorted(np.random.default_rng(T).choice(256, 12, replace=False).tolist())
    o, s, o_ref, s_ref = _run(inp, batches=rows)
    check("o", o[rows], o_ref[rows], torch.bfloat16)
    check("state", s[rows], s_ref[rows], torch.bfloat16)
    _ulp_consistent(s[rows], s_ref[rows])
    # every row's state was rewritten (alpha < 1 almost surely changes the bits)
    assert not torch.equal(s[200], inp.state[200])


def test_decode_empty_batch():
    inp = workloads.make_decode(1, 1, 2, 4, 128, 128, seed=64)
    state = inp.state.to(DEV)
    z = lambda t: t[:0].to(DEV)
    o = binding.gdn_decode(z(inp.q), z(inp.k), z(inp.v), z(inp.a), z(inp.b), inp.A_log.to(DEV),
                           inp.dt_bias.to(DEV), state)
    torch.cuda.synchronize()
    assert o.shape[0] == 0


@pytest.mark.parametrize("sp_beta", [1.0, 2.0])
@pytest.mark.parametrize("T", [1, 3])
def test_decode_softplus_threshold(T, sp_beta):
    """Gate inputs on both sides of the softplus threshold: per v-head,
    dt_bias puts softplus_beta * (a + dt_bias) well above, just above, just
    below and well below the threshold of 20 (a ~ N(0, 1) in bf16), in the
    per-token kernel (T = 1) and the closed-form kernel (T = 3); softplus_beta
    = 2 moves the switch to x = 10.  Small A_log keeps the decay of the
    linear branch (g = -exp(A_log) * x) inside fp32 range."""
    print(f"decode softplus T={T} sp_beta={sp_beta}", flush=True)
    inp = workloads.make_decode(5, T, 2, 8, 128, 128, seed=90 + T)
    thr_x = 20.0 / sp_beta
    inp.dt_bias = torch.tensor([thr_x + d for d in (6.0, 1.5, 0.25, -0.25, -1.5, -6.0, 0.0, -thr_x)],
                               dtype=torch.float32)
    inp.A_log = torch.full((8,), -3.0, dtype=torch.float32)
    x = inp.a.float() + inp.dt_bias
    above = (sp_beta * x > 20.0).float().mean().item()
    assert 0.2 < above < 0.8, f"threshold not straddled ({above:.2f} above)"
    o, s, o_ref, s_ref = _run(inp, sp_beta=sp_beta)
    check("o", o, o_ref, torch.bfloat16)
    check("state", s, s_ref, torch.bfloat16)
    _ulp_consistent(s, s_ref)
