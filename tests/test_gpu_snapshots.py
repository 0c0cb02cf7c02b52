"""GPU parity of the state snapshots (h_snap every split_size tokens) of the
GDN and KDA chunked prefill against the fp64 oracle, through the C ABI, on
all four scan paths (bf16 / fp32 io, scalar / per-channel gate)."""

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_61_amd import binding, workloads
from tests.tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
dv = lambda t: None if t is None else t.to(DEV)


def _gdn(inp, S, fp32_states=False):
    print(f"snapshots GDN {inp.name} dims={inp.dims} split={S} fp32 states={fp32_states}", flush=True)
    o, ht, hs = binding.gdn_chunk_fwd(dv(inp.q), dv(inp.k), dv(inp.v), dv(inp.g), dv(inp.beta),
                                      scale=inp.scale, h0=dv(inp.h0), cu_seqlens=dv(inp.cu_seqlens),
                                      split_size=S, states_in_fp32=fp32_states, cu_seqlens_cpu=inp.cu_seqlens)
    assert hs.dtype == (torch.float32 if fp32_states or inp.q.dtype == torch.float32 else torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, ht_ref, hs_ref = oracle.gdn_recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale,
                                                 h0=inp.h0, cu_seqlens=inp.cu_seqlens, split_size=S)
    assert hs.shape == hs_ref.shape
    dt = inp.q.dtype
    check("o", o.cpu(), o_ref, dt)
    check("ht", ht.cpu(), ht_ref, dt)
    print("  h_snap", check("h_snap", hs.cpu(), hs_ref, dt), flush=True)


def _kda(inp, S, fp32_states=False):
    print(f"snapshots KDA {inp.name} dims={inp.dims} split={S} fp32 states={fp32_states}", flush=True)
    o, ht, _, _, hs = binding.kda_chunk_fwd(dv(inp.q), dv(inp.k), dv(inp.v), dv(inp.gk), dv(inp.beta),
                                            scale=inp.scale, h0=dv(inp.h0), cu_seqlens=dv(inp.cu_seqlens),
                                            return_intra=False, split_size=S, states_in_fp32=fp32_states,
                                            cu_seqlens_cpu=inp.cu_seqlens)
    torch.cuda.synchronize()
    o_ref, ht_ref, hs_ref = oracle.kda_recurrent(inp.q, inp.k, inp.v, inp.gk, inp.beta, inp.scale,
                                                 h0=inp.h0, cu_seqlens=inp.cu_seqlens, split_size=S)
    assert hs.shape == hs_ref.shape
    dt = inp.q.dtype
    check("o", o.cpu(), o_ref, dt)
    print("  h_snap", check("h_snap", hs.cpu(), hs_ref, dt), flush=True)


@pytest.mark.parametrize("fp32_states", [False, True])
@pytest.mark.parametrize("S", [64, 128])
def test_gdn_bf16_varlen_snapshots(S, fp32_states):
    inp = workloads.make_prefill(1, 400, 2, 4, 128, 128, dtype=torch.bfloat16, seed=S, h0=True,
                                 seqlens=[130, 64, 1, 205], name="bf16_varlen")
    _gdn(inp, S, fp32_states)


@pytest.mark.parametrize("fp32_states", [False, True])
@pytest.mark.parametrize("S", [64, 128])
def test_gdn_bf16_snapshots_64_column_work_groups(S, fp32_states):
    # 3 x 16 (q / k head) units x 2 v-heads: the 64-column scan
    inp = workloads.make_prefill(3, 260, 16, 32, 128, 128, dtype=torch.bfloat16, seed=510 + S, h0=True,
                                 name="bf16_64col_snap")
    _gdn(inp, S, fp32_states)


@pytest.mark.parametrize("N,K,hi", [(150, 128, 100), (150, 64, 100), (1100, 64, 3)],
                         ids=["150seqs_K128", "150seqs_K64", "1100seqs_tiny"])
def test_gdn_many_sequences_with_snapshots(N, K, hi):
    # snapshot offsets summed over many earlier sequences (more than one
    # 64-lane stride), chunk tables and the longest-first order for N <= 1024
    # and beyond it; lengths 0 .. hi, empty sequences included
    lens = workloads.draw_seqlens(N, 0, hi, seed=520 + N + K)
    inp = workloads.make_prefill(1, sum(lens), 1, 2, K, K, dtype=torch.bfloat16, seed=521 + N, h0=True,
                                 seqlens=lens, name=f"many{N}_K{K}")
    _gdn(inp, 64)


def test_kda_many_sequences_with_snapshots():
    lens = workloads.draw_seqlens(150, 0, 100, seed=530)
    inp = workloads.make_prefill(1, sum(lens), 1, 1, 128, 128, dtype=torch.bfloat16, seed=531, gate="kda",
                                 h0=True, seqlens=lens, name="kda_many150")
    _kda(inp, 64)


def test_gdn_bf16_fixed_snapshots_every_chunk():
    inp = workloads.make_prefill(2, 200, 1, 2, 64, 64, dtype=torch.bfloat16, seed=5, h0=True,
                                 name="bf16_K64")
    _gdn(inp, 64)


def test_gdn_fp32_snapshots():
    inp = workloads.make_prefill(2, 150, 1, 2, 64, 64, dtype=torch.float32, seed=6, h0=True,
                                 name="fp32_K64")
    _gdn(inp, 64)


@pytest.mark.parametrize("fp32_states", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kda_snapshots(dtype, fp32_states):
    inp = workloads.make_prefill(1, 260, 2, 2, 128, 128, dtype=dtype, seed=7, gate="kda", h0=True,
                                 seqlens=[70, 190], name=f"kda_{dtype}")
    _kda(inp, 128 if dtype == torch.bfloat16 else 64, fp32_states)


def test_snapshot_buffer_untouched_without_snapshots():
    """split_size given but the call has no tokens: no snapshot exists."""
    inp = workloads.make_prefill(1, 64, 1, 2, 64, 64, dtype=torch.bfloat16, seed=8, h0=True,
                                 seqlens=[0, 64], name="empty_first")
    _gdn(inp, 64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gdn_g_gamma(dtype):
    """Fixed per-head decay in place of g (varlen, h0, GQA)."""
    inp = workloads.make_prefill(1, 300, 2, 4, 64, 64, dtype=dtype, seed=9, h0=True,
                                 seqlens=[100, 200], name=f"gamma_{dtype}")
    gamma = torch.tensor([-0.02, -0.1, -0.5, -2.0], dtype=torch.float32)
    print(f"g_gamma {dtype}", flush=True)
    o, ht = binding.gdn_chunk_fwd(dv(inp.q), dv(inp.k), dv(inp.v), None, dv(inp.beta), scale=inp.scale,
                                  h0=dv(inp.h0), cu_seqlens=dv(inp.cu_seqlens), g_gamma=dv(gamma))
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.gdn_recurrent(inp.q, inp.k, inp.v, None, inp.beta, inp.scale, h0=inp.h0,
                                         cu_seqlens=inp.cu_seqlens, g_gamma=gamma)
    check("o", o.cpu(), o_ref, dtype)
    check("ht", ht.cpu(), ht_ref, dtype)


def test_snapshots_b4_t4096_sampled_heads():
    """The headline workload (B=4 T=4096 H=16 K=V=128) with snapshots every 64
    tokens, as bench.py times it: two sampled heads of every sequence."""
    inp = workloads.gdn_bf16_b4_t4096()
    heads = [3, 12]
    print(f"snapshots full size heads={heads}", flush=True)
    o, ht, hs = binding.gdn_chunk_fwd(dv(inp.q), dv(inp.k), dv(inp.v), dv(inp.g), dv(inp.beta),
                                      scale=inp.scale, split_size=64, states_in_fp32=True)
    torch.cuda.synchronize()
    _, ht_ref, hs_ref = oracle.gdn_recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale,
                                             heads=heads, split_size=64)
    hs = hs.cpu()
    print("  h_snap", check("h_snap", hs[:, heads], hs_ref[:, heads], torch.bfloat16), flush=True)
    check("ht", ht.cpu()[:, heads], ht_ref[:, heads], torch.bfloat16)


def test_snapshot_capacity_bounds_varlen_writes():
    """A varlen call whose snapshot buffer holds fewer entries than the call
    has: the entries within the capacity are the oracle's, the guard rows
    after them are untouched (no write past the capacity)."""
    inp = workloads.make_prefill(1, 400, 2, 4, 64, 64, dtype=torch.bfloat16, seed=11, h0=True,
                                 seqlens=[130, 64, 1, 205], name="bf16_varlen_cap")
    S, cap = 64, 5                   # the call has 3 + 1 + 1 + 4 = 9 snapshots
    buf = torch.full((cap + 3, 4, 64, 64), 7.0, dtype=torch.float32, device=DEV)
    print("snapshot capacity", flush=True)
    o, ht, hs = binding.gdn_chunk_fwd(dv(inp.q), dv(inp.k), dv(inp.v), dv(inp.g), dv(inp.beta),
                                      scale=inp.scale, h0=dv(inp.h0), cu_seqlens=dv(inp.cu_seqlens),
                                      split_size=S, h_snap=buf[:cap], states_in_fp32=True)
    torch.cuda.synchronize()
    _, _, hs_ref = oracle.gdn_recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0,
                                        cu_seqlens=inp.cu_seqlens, split_size=S)
    assert hs_ref.shape[0] == 9
    got = buf.cpu()
    check("h_snap", got[:cap], hs_ref[:cap], torch.bfloat16)
    assert torch.all(got[cap:] == 7.0), "entries past the capacity were written"
