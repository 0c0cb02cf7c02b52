"""GPU parity of the forward decay-only state scan (gdn_chunk_fwd_h, C ABI)
against the fp64 oracle: the state at the start of every split and the final
state, for every gate form (scalar, fixed per-head, per key channel, per
value channel, scalar with per value channel, none), ragged and empty
sequences, GQA heads, an initial state, K = V = 64 and 128."""

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_61_amd import binding, workloads
from tests.tolerance import STATE_SCAN_REL, check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
dv = lambda t: None if t is None else t.to(DEV)


def _gates(inp, gate, rng):
    B, T, Hk, HV, K, V = inp.dims
    forms = (gate or "").split("+")
    g = inp.g if "gdn" in forms else None
    gk = inp.gk if "kda" in forms else None
    gamma = torch.from_numpy(-np.abs(rng.standard_normal(HV)).astype(np.float32) * 0.05) if "gamma" in forms else None
    gv = None
    if "gv" in forms:   # per-value-channel log-gates, -softplus(N(0, 1)) * 0.05
        gv = torch.from_numpy((-np.logaddexp(0, rng.standard_normal((B, T, HV, V))) * 0.05).astype(np.float32))
    return g, gamma, gk, gv


def _rel(t):
    """fp32-stored states: the state scans' tight bar; bf16-stored: the bf16 bar."""
    return STATE_SCAN_REL if t.dtype == torch.float32 else None


def _case(inp, gate, S, seed=0, fp32_states=False, v_first=True):
    """``v_first=False``: h0 goes in, and h / ht come out, as [*, HV, K, V];
    they are transposed back for the comparison."""
    rng = np.random.default_rng(seed)
    g, gamma, gk, gv = _gates(inp, gate, rng)
    print(f"fwd h {inp.name} gate={gate} split={S} dims={inp.dims} h0={inp.h0 is not None} "
          f"fp32 states={fp32_states} v_first={v_first}", flush=True)
    lay = (lambda x: x) if v_first else (lambda x: None if x is None else x.transpose(-1, -2).contiguous())
    h, ht = binding.chunk_fwd_h(dv(inp.k), dv(inp.v), g=dv(g), g_gamma=dv(gamma), gk=dv(gk), gv=dv(gv),
                                h0=dv(lay(inp.h0)), cu_seqlens=dv(inp.cu_seqlens), split_size=S,
                                states_in_fp32=fp32_states, cu_seqlens_cpu=inp.cu_seqlens, state_v_first=v_first)
    torch.cuda.synchronize()
    h, ht = lay(h), lay(ht)
    assert h.dtype == (torch.float32 if fp32_states else torch.bfloat16)
    h_ref, ht_ref = oracle.state_scan(inp.k, inp.v, g=g, g_gamma=gamma, gk=gk, gv=gv, h0=inp.h0,
                                      cu_seqlens=inp.cu_seqlens, split_size=S)
    assert h.shape == h_ref.shape
    h = h.cpu()
    print("  h", check("h", h, h_ref, torch.bfloat16, rel=_rel(h)),
          " ht", check("ht", ht.cpu(), ht_ref, torch.bfloat16, rel=STATE_SCAN_REL), flush=True)


@pytest.mark.parametrize("fp32_states", [False, True])
@pytest.mark.parametrize("gate", ["gdn", "gamma", None, "gv", "gdn+gv", "gamma+gv"])
def test_fwd_h_varlen_gqa(gate, fp32_states):
    inp = workloads.make_prefill(1, 331, 2, 4, 128, 128, dtype=torch.bfloat16, seed=70, h0=True,
                                 seqlens=[200, 1, 0, 130], name="fwd_h_varlen")
    _case(inp, gate, 64, seed=71, fp32_states=fp32_states)


@pytest.mark.parametrize("fp32_states", [False, True])
@pytest.mark.parametrize("gate", ["gdn", "gamma", None, "gv", "gdn+gv", "kda"])
def test_fwd_h_key_first_layout(gate, fp32_states):
    """The page's default state layout ([*, HV, K, V], V contiguous) for h0,
    h and ht, in each of the three kernels (scalar / no gate, gv, gk)."""
    inp = workloads.make_prefill(1, 331, 2, 4, 128, 128, dtype=torch.bfloat16, seed=83, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=[200, 1, 0, 130],
                                 name="fwd_h_kfirst")
    _case(inp, gate, 64, seed=84, fp32_states=fp32_states, v_first=False)


@pytest.mark.parametrize("gate", ["gdn", "gv", "kda"])
def test_fwd_h_many_sequences(gate):
    """150 packed sequences of 0..100 tokens: stored-state offsets summed over
    many earlier sequences, in each of the three kernels."""
    lens = workloads.draw_seqlens(150, 0, 100, seed=540)
    inp = workloads.make_prefill(1, sum(lens), 1, 2, 128, 128, dtype=torch.bfloat16, seed=541, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=lens, name="fwd_h_many150")
    _case(inp, gate, 64, seed=542, fp32_states=True)


@pytest.mark.parametrize("gate", ["gdn", "gv", "kda"])
def test_fwd_h_key_first_k64(gate):
    inp = workloads.make_prefill(2, 150, 1, 2, 64, 64, dtype=torch.bfloat16, seed=85, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", name="fwd_h_kfirst_K64")
    _case(inp, gate, 128, seed=86, v_first=False)


@pytest.mark.parametrize("gate", ["gdn", "gv", "gdn+gv", "kda"])
def test_fwd_h_k64(gate):
    inp = workloads.make_prefill(2, 150, 1, 2, 64, 64, dtype=torch.bfloat16, seed=72,
                                 gate="kda" if gate == "kda" else "gdn", name="fwd_h_K64")
    _case(inp, gate, 128, seed=73)


@pytest.mark.parametrize("fp32_states", [False, True])
def test_fwd_h_kda_k128_varlen(fp32_states):
    inp = workloads.make_prefill(1, 200, 2, 2, 128, 128, dtype=torch.bfloat16, seed=74, gate="kda", h0=True,
                                 seqlens=[64, 136], name="fwd_h_kda_K128")
    _case(inp, "kda", 64, seed=75, fp32_states=fp32_states)


def test_fwd_h_final_state_only():
    inp = workloads.make_prefill(2, 100, 2, 2, 128, 128, dtype=torch.bfloat16, seed=76, h0=True, name="fwd_h_ht")
    h, ht = binding.chunk_fwd_h(dv(inp.k), dv(inp.v), g=dv(inp.g), h0=dv(inp.h0), split_size=None)
    torch.cuda.synchronize()
    assert h is None
    _, ht_ref = oracle.state_scan(inp.k, inp.v, g=inp.g, h0=inp.h0)
    check("ht", ht.cpu(), ht_ref, torch.bfloat16, rel=STATE_SCAN_REL)


def test_fwd_h_b4_t4096_sampled_heads():
    """The shape bench.py times (B=4 T=4096 H=16 K=V=128, scalar gate, h at
    every chunk, ht out): two sampled heads, every chunk of every sequence."""
    inp = workloads.gdn_bf16_b4_t4096()
    heads = [0, 13]
    print(f"fwd h full size heads={heads}", flush=True)
    h, ht = binding.chunk_fwd_h(dv(inp.k), dv(inp.v), g=dv(inp.g), split_size=64, states_in_fp32=True)
    torch.cuda.synchronize()
    # Hk = HV here: v-head h reads k head h
    h_ref, ht_ref = oracle.state_scan(inp.k[:, :, heads], inp.v[:, :, heads], g=inp.g[:, :, heads], split_size=64)
    check("h", h.cpu()[:, heads], h_ref, torch.bfloat16, rel=STATE_SCAN_REL)
    check("ht", ht.cpu()[:, heads], ht_ref, torch.bfloat16, rel=STATE_SCAN_REL)


@pytest.mark.parametrize("gate", ["gamma+gv", "kda"])
def test_fwd_h_split_of_three_chunks(gate):
    """split_size = 192 (a stored state every third chunk), odd lengths, GQA."""
    inp = workloads.make_prefill(1, 455, 1, 2, 64, 64, dtype=torch.bfloat16, seed=77, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=[390, 0, 65], name="fwd_h_split192")
    _case(inp, gate, 192, seed=78)


def test_fwd_h_b4_t4096_bf16_states_sampled_heads():
    """The same shape with the page's default storage (states in the input
    dtype, bf16): two sampled heads."""
    inp = workloads.gdn_bf16_b4_t4096()
    heads = [5, 10]
    print(f"fwd h full size bf16 states heads={heads}", flush=True)
    h, ht = binding.chunk_fwd_h(dv(inp.k), dv(inp.v), g=dv(inp.g), split_size=64)
    torch.cuda.synchronize()
    assert h.dtype == torch.bfloat16
    h_ref, ht_ref = oracle.state_scan(inp.k[:, :, heads], inp.v[:, :, heads], g=inp.g[:, :, heads], split_size=64)
    check("h", h.cpu()[:, heads], h_ref, torch.bfloat16)
    check("ht", ht.cpu()[:, heads], ht_ref, torch.bfloat16, rel=STATE_SCAN_REL)


@pytest.mark.parametrize("gate", ["gdn", "kda", "gamma+gv"])
def test_fwd_h_grouped_gate_heads(gate):
    """Gates of Hg = 2 heads shared by HV = 4 v-heads (gate head j // 2)."""
    inp = workloads.make_prefill(1, 300, 4, 4, 64, 64, dtype=torch.bfloat16, seed=81, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=[170, 130], name="fwd_h_grouped")
    rng = np.random.default_rng(82)
    g, gamma, gk, gv = _gates(inp, gate, rng)
    cut = lambda x, ax: None if x is None else x.narrow(ax, 0, 2).contiguous()
    g, gk, gv, gamma = cut(g, 2), cut(gk, 2), cut(gv, 2), cut(gamma, 0)
    print(f"fwd h grouped gates {gate}", flush=True)
    h, ht = binding.chunk_fwd_h(dv(inp.k), dv(inp.v), g=dv(g), g_gamma=dv(gamma), gk=dv(gk), gv=dv(gv),
                                h0=dv(inp.h0), cu_seqlens=dv(inp.cu_seqlens), split_size=128,
                                states_in_fp32=True, cu_seqlens_cpu=inp.cu_seqlens)
    torch.cuda.synchronize()
    h_ref, ht_ref = oracle.state_scan(inp.k, inp.v, g=g, g_gamma=gamma, gk=gk, gv=gv, h0=inp.h0,
                                      cu_seqlens=inp.cu_seqlens, split_size=128)
    check("h", h.cpu(), h_ref, torch.bfloat16, rel=STATE_SCAN_REL)
    check("ht", ht.cpu(), ht_ref, torch.bfloat16, rel=STATE_SCAN_REL)


# the scalar-gate kernel's ring of four LDS slots (loads three chunks ahead)
# and its loop unrolled by four: sequences of 0, 1, 2, ..., 8, 9 and 10 chunks
# with ragged tails, both key widths, bf16 and fp32 stored states
RING_LENS = [0, 1, 65, 130, 255, 320, 384, 448, 512, 513, 577]


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("S,fp32_states", [(64, False), (128, True)])
@pytest.mark.parametrize("gate", ["gdn", "gamma"])
def test_fwd_h_ring_chunk_counts(K, S, fp32_states, gate):
    inp = workloads.make_prefill(1, sum(RING_LENS), 2, 4, K, K, dtype=torch.bfloat16, seed=90 + K, h0=True,
                                 seqlens=RING_LENS, name="fwd_h_ring")
    _case(inp, gate, S, seed=93, fp32_states=fp32_states)
