"""GPU parity at sizes whose tensors pass 4 GiB, so that element and byte
offsets into them need more than 32 bits: the bf16 GDN prefill with q, k, v
and o of 4.56 GB each, the intra-chunk step with k, v, w and u of 4.56 GB
each, the forward state scan with fp32 states stored every
chunk (4.56 GB), and decode and the handoff on a bf16 state pool of 8.6 GB.

Only a few heads or pool slots carry seeded random data (among them the
last, at the highest offsets); the oracle checks those one by one.  Every
other head is zero input and must come out exactly zero, and every other
slot must stay untouched: a wrapped offset that lands anywhere else in the
tensor breaks that."""

import gc

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_61_amd import binding, workloads
from tests.tolerance import STATE_SCAN_REL, check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
T_BIG = 139264       # 2176 chunks; T x 128 heads x 128 bf16 values = 4.56 GB
POOL_BIG = 8200      # 8200 x 32 heads x 128 x 128 bf16 = 8.6 GB


def _zeros(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def _release():
    gc.collect()
    torch.cuda.empty_cache()


def _heads(T, heads, tag, seed0):
    """One seeded single-head problem per sampled head."""
    return {j: workloads.make_prefill(1, T, 1, 1, 128, 128, dtype=torch.bfloat16, seed=seed0 + i, h0=True,
                                      name=f"{tag}_head{j}")
            for i, j in enumerate(heads)}


def test_gdn_prefill_offsets_past_4gib():
    H, K, T = 128, 128, T_BIG
    small = _heads(T, (0, H - 1), "big_prefill", 301)
    print(f"prefill offsets past 4 GiB: B=1 T={T} Hk=HV={H} K=V={K} bf16, sampled heads {list(small)}",
          flush=True)
    q, k, v = _zeros(1, T, H, K), _zeros(1, T, H, K), _zeros(1, T, H, K)
    g, beta = _zeros(1, T, H, dtype=torch.float32), _zeros(1, T, H, dtype=torch.float32)
    h0 = _zeros(1, H, K, K, dtype=torch.float32)
    for j, s in small.items():
        for dst, src in ((q, s.q), (k, s.k), (v, s.v)):
            dst[:, :, j] = src[:, :, 0].to(DEV)
        g[:, :, j] = s.g[:, :, 0].to(DEV)
        beta[:, :, j] = s.beta[:, :, 0].to(DEV)
        h0[:, j] = s.h0[:, 0].to(DEV)
    assert v.numel() * v.element_size() > 1 << 32
    o, ht = binding.gdn_chunk_fwd(q, k, v, g, beta, scale=K ** -0.5, h0=h0)
    torch.cuda.synchronize()
    del q, k, v, g, beta
    for j, s in small.items():
        o_ref, ht_ref = oracle.gdn_recurrent(s.q, s.k, s.v, s.g, s.beta, s.scale, h0=s.h0)
        print(f"  head {j}: o", check("o", o[:, :, j:j + 1].cpu(), o_ref, torch.bfloat16),
              " ht", check("ht", ht[:, j:j + 1].cpu(), ht_ref, torch.bfloat16), flush=True)
        o[:, :, j] = 0
        ht[:, j] = 0
    assert not bool(torch.any(o != 0)), "output written outside the sampled heads"
    assert not bool(torch.any(ht != 0)), "final state written outside the sampled heads"
    del o, ht, h0
    _release()


def test_chunk_intra_offsets_past_4gib():
    H, K, T = 128, 128, T_BIG
    small = _heads(T, (0, H - 1), "big_intra", 311)
    print(f"intra w/u offsets past 4 GiB: B=1 T={T} Hk=HV={H} K=V={K} bf16, sampled heads {list(small)}",
          flush=True)
    k, v = _zeros(1, T, H, K), _zeros(1, T, H, K)
    g, beta = _zeros(1, T, H, dtype=torch.float32), _zeros(1, T, H, dtype=torch.float32)
    for j, s in small.items():
        k[:, :, j] = s.k[:, :, 0].to(DEV)
        v[:, :, j] = s.v[:, :, 0].to(DEV)
        g[:, :, j] = s.g[:, :, 0].to(DEV)
        beta[:, :, j] = s.beta[:, :, 0].to(DEV)
    w, u, A = binding.gdn_chunk_intra(k, v, g, beta)
    torch.cuda.synchronize()
    assert w.numel() * w.element_size() > 1 << 32
    del k, v, g, beta
    # zero heads: beta 0 gives A = I, w = u = 0
    eye = (torch.arange(64, device=DEV)[None, :] == (torch.arange(T, device=DEV) % 64)[:, None]).to(A.dtype)
    for j, s in small.items():
        A_ref, w_ref, u_ref = oracle.chunk_intra_wu(s.k, s.v, s.beta, g=s.g)
        print(f"  head {j}:", check("A", A[:, :, j:j + 1].cpu(), A_ref, torch.bfloat16),
              check("w", w[:, :, j:j + 1].cpu(), w_ref, torch.bfloat16),
              check("u", u[:, :, j:j + 1].cpu(), u_ref, torch.bfloat16), flush=True)
        w[:, :, j] = 0
        u[:, :, j] = 0
        A[0, :, j] = eye
    assert not bool(torch.any(w != 0)), "w written outside the sampled heads"
    assert not bool(torch.any(u != 0)), "u written outside the sampled heads"
    assert bool(torch.all(A == eye[None, :, None, :])), "A written outside the sampled heads"
    del w, u, A, eye
    _release()


def test_fwd_h_states_past_4gib():
    HV, K, T = 32, 128, T_BIG
    small = _heads(T, (0, HV - 1), "big_fwd_h", 311)
    print(f"fwd_h states past 4 GiB: B=1 T={T} Hk=HV={HV} K=V={K}, fp32 states every chunk, "
          f"sampled heads {list(small)}", flush=True)
    k, v = _zeros(1, T, HV, K), _zeros(1, T, HV, K)
    g = _zeros(1, T, HV, dtype=torch.float32)
    h0 = _zeros(1, HV, K, K, dtype=torch.float32)
    for j, s in small.items():
        k[:, :, j] = s.k[:, :, 0].to(DEV)
        v[:, :, j] = s.v[:, :, 0].to(DEV)
        g[:, :, j] = s.g[:, :, 0].to(DEV)
        h0[:, j] = s.h0[:, 0].to(DEV)
    h, ht = binding.chunk_fwd_h(k, v, g=g, h0=h0, split_size=64, states_in_fp32=True)
    torch.cuda.synchronize()
    assert h.dtype == torch.float32 and h.numel() * 4 > 1 << 32
    del k, v, g
    for j, s in small.items():
        h_ref, ht_ref = oracle.state_scan(s.k, s.v, g=s.g, h0=s.h0, split_size=64)
        print(f"  head {j}: h", check("h", h[:, j:j + 1].cpu(), h_ref, torch.bfloat16, rel=STATE_SCAN_REL),
              " ht", check("ht", ht[:, j:j + 1].cpu(), ht_ref, torch.bfloat16, rel=STATE_SCAN_REL), flush=True)
        h[:, j] = 0
        ht[:, j] = 0
    assert not bool(torch.any(h != 0)), "states written outside the sampled heads"
    assert not bool(torch.any(ht != 0)), "final state written outside the sampled heads"
    del h, ht, h0
    _release()


@pytest.mark.parametrize("T", [1, 3])
def test_decode_pool_past_4gib(T):
    B, H, HV, K = 4, 16, 32, 128
    slots = [POOL_BIG - 1, 4100, 17, POOL_BIG - 2]
    print(f"decode pool past 4 GiB: B={B} T={T} H={H} HV={HV} pool={POOL_BIG} slots={slots}", flush=True)
    dec = workloads.make_decode(B, T, H, HV, K, K, seed=320 + T)
    ps = _zeros(POOL_BIG, HV, K, K)
    assert ps.numel() * 2 > 1 << 33
    for b, sl in enumerate(slots):
        ps[sl] = dec.state[b].to(DEV)
    d = lambda t: t.to(DEV)
    o = binding.gdn_decode(d(dec.q), d(dec.k), d(dec.v), d(dec.a), d(dec.b), d(dec.A_log), d(dec.dt_bias), ps,
                           torch.tensor(slots, dtype=torch.int32, device=DEV), scale=dec.scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gdn_decode(dec.q, dec.k, dec.v, dec.a, dec.b, dec.A_log, dec.dt_bias, dec.state,
                                     scale=dec.scale)
    got = torch.stack([ps[sl] for sl in slots]).cpu()
    print("  o", check("o", o.cpu(), o_ref, torch.bfloat16), " state", check("state", got, s_ref, torch.bfloat16),
          flush=True)
    for sl in slots:
        ps[sl] = 0
    assert not bool(torch.any(ps != 0)), "pool written outside the batch's slots"
    del ps
    _release()


def test_state_to_pool_past_4gib():
    N, HV, K = 3, 32, 128
    slots = [POOL_BIG - 1, 0, 6000]
    print(f"handoff pool past 4 GiB: N={N} HV={HV} pool={POOL_BIG} slots={slots}", flush=True)
    rng = np.random.default_rng(330)
    ht = rng.standard_normal((N, HV, K, K)).astype(np.float32) * 0.3
    ps = _zeros(POOL_BIG, HV, K, K)
    binding.state_to_pool(torch.from_numpy(ht).to(DEV), ps, torch.tensor(slots, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    # the oracle's handoff into a pool of N slots in order: the same roundings
    want = oracle.state_to_pool(ht, np.zeros((N, HV, K, K)), list(range(N)))
    got = torch.stack([ps[sl] for sl in slots]).cpu().double().numpy()
    assert np.array_equal(got, want)
    for sl in slots:
        ps[sl] = 0
    assert not bool(torch.any(ps != 0)), "pool written outside the given slots"
    del ps
    _release()
