"""GPU parity of the backward state-gradient scan (gdn_chunk_bwd_dh, C ABI)
against the fp64 oracle: dh every split_size tokens and dh0, for the scalar
gate, the fixed per-head decay, the per-key-channel gate, the per-value-channel
gate (alone and with a scalar gate) and no gate."""

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_61_amd import binding, workloads
from tests.tolerance import STATE_SCAN_REL, check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
dv = lambda t: None if t is None else t.to(DEV)


def _case(inp, gate, S, dht_std=0.1, seed=0, fp32_states=False, gate_heads=None, v_first=True):
    """``v_first=False``: dht goes in, and dh / dh0 come out, as
    [*, HV, K, V]; they are transposed back for the comparison."""
    B, T, Hk, HV, K, V = inp.dims
    rng = np.random.default_rng(seed)
    do = torch.from_numpy(rng.standard_normal((B, T, HV, V)).astype(np.float32)).to(torch.bfloat16)
    N = inp.num_seqs
    dht = torch.from_numpy((rng.standard_normal((N, HV, V, K)) * dht_std).astype(np.float32))
    forms = (gate or "").split("+")
    g = inp.g if "gdn" in forms else None
    gk = inp.gk if "kda" in forms else None
    gamma = torch.from_numpy(-np.abs(rng.standard_normal(HV)).astype(np.float32) * 0.05) if "gamma" in forms else None
    gv = None
    if "gv" in forms:   # per-value-channel log-gates, -softplus(N(0, 1)) * 0.05
        gv = torch.from_numpy((-np.logaddexp(0, rng.standard_normal((B, T, HV, V))) * 0.05).astype(np.float32))
    if gate_heads is not None:   # gates of fewer heads, shared by HV // gate_heads v-heads
        cut = lambda x, ax: None if x is None else x.narrow(ax, 0, gate_heads).contiguous()
        g, gk, gv, gamma = cut(g, 2), cut(gk, 2), cut(gv, 2), cut(gamma, 0)
    print(f"bwd dh {inp.name} gate={gate} split={S} dims={inp.dims} fp32 states={fp32_states} "
          f"gate heads={gate_heads} v_first={v_first}", flush=True)
    lay = (lambda x: x) if v_first else (lambda x: None if x is None else x.transpose(-1, -2).contiguous())
    dh, dh0 = binding.chunk_bwd_dh(dv(inp.q), dv(do), g=dv(g), g_gamma=dv(gamma), gk=dv(gk), gv=dv(gv),
                                   scale=inp.scale, dht=dv(lay(dht)), cu_seqlens=dv(inp.cu_seqlens), split_size=S,
                                   states_in_fp32=fp32_states, cu_seqlens_cpu=inp.cu_seqlens,
                                   state_v_first=v_first)
    torch.cuda.synchronize()
    dh, dh0 = lay(dh), lay(dh0)
    assert dh.dtype == (torch.float32 if fp32_states else torch.bfloat16)
    dh_ref, dh0_ref = oracle.state_grad_scan(inp.q, do, inp.scale, g=g, g_gamma=gamma, gk=gk, gv=gv, dht=dht,
                                             cu_seqlens=inp.cu_seqlens, split_size=S)
    assert dh.shape == dh_ref.shape
    dh = dh.cpu()
    print("  dh", check("dh", dh, dh_ref, torch.bfloat16, rel=STATE_SCAN_REL if fp32_states else None),
          " dh0", check("dh0", dh0.cpu(), dh0_ref, torch.bfloat16, rel=STATE_SCAN_REL), flush=True)


@pytest.mark.parametrize("fp32_states", [False, True])
@pytest.mark.parametrize("gate", ["gdn", "gamma", None, "gv", "gdn+gv", "gamma+gv"])
def test_bwd_dh_scalar_gate_varlen(gate, fp32_states):
    inp = workloads.make_prefill(1, 330, 2, 4, 128, 128, dtype=torch.bfloat16, seed=60, h0=True,
                                 seqlens=[200, 1, 129], name="bwd_varlen")
    _case(inp, gate, 64, seed=61, fp32_states=fp32_states)


@pytest.mark.parametrize("fp32_states", [False, True])
@pytest.mark.parametrize("gate", ["gdn", "gamma", None, "gv", "gamma+gv", "kda"])
def test_bwd_dh_key_first_layout(gate, fp32_states):
    """The page's default state layout ([*, HV, K, V], V contiguous) for
    dht, dh and dh0, in each of the three kernels (scalar / no gate, gv, gk)."""
    inp = workloads.make_prefill(1, 330, 2, 4, 128, 128, dtype=torch.bfloat16, seed=68, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=[200, 1, 129],
                                 name="bwd_kfirst")
    _case(inp, gate, 64, seed=69, fp32_states=fp32_states, v_first=False)


@pytest.mark.parametrize("gate", ["gamma", "gdn+gv", "kda"])
def test_bwd_dh_key_first_k64(gate):
    inp = workloads.make_prefill(2, 150, 1, 2, 64, 64, dtype=torch.bfloat16, seed=87,
                                 gate="kda" if gate == "kda" else "gdn", name="bwd_kfirst_K64")
    _case(inp, gate, 128, seed=88, v_first=False)


@pytest.mark.parametrize("gate", ["gv", "gdn+gv"])
def test_bwd_dh_gv_k64(gate):
    inp = workloads.make_prefill(2, 150, 1, 2, 64, 64, dtype=torch.bfloat16, seed=67, name="bwd_gv_K64")
    _case(inp, gate, 128, seed=68)


def test_bwd_dh_kda():
    inp = workloads.make_prefill(2, 150, 1, 2, 64, 64, dtype=torch.bfloat16, seed=62, gate="kda",
                                 name="bwd_kda_K64")
    _case(inp, "kda", 128, seed=63)


@pytest.mark.parametrize("fp32_states", [False, True])
def test_bwd_dh_kda_k128_varlen(fp32_states):
    inp = workloads.make_prefill(1, 200, 2, 2, 128, 128, dtype=torch.bfloat16, seed=64, gate="kda",
                                 seqlens=[64, 136], name="bwd_kda_K128")
    _case(inp, "kda", 64, seed=65, fp32_states=fp32_states)


def test_bwd_dh_b4_t4096_sampled_heads():
    """The shape bench.py times (B=4 T=4096 H=16 K=V=128, scalar gate, dh every
    chunk, dht in): two sampled heads, every chunk of every sequence."""
    inp = workloads.gdn_bf16_b4_t4096()
    B, T, Hk, HV, K, V = inp.dims
    rng = np.random.default_rng(66)
    heads = [0, 9]
    do = torch.from_numpy(rng.standard_normal((B, T, HV, V)).astype(np.float32)).to(torch.bfloat16)
    dht = torch.from_numpy((rng.standard_normal((B, HV, V, K)) * 0.1).astype(np.float32))
    print(f"bwd dh full size heads={heads}", flush=True)
    dh, dh0 = binding.chunk_bwd_dh(dv(inp.q), dv(do), g=dv(inp.g), scale=inp.scale, dht=dv(dht), split_size=64,
                                   states_in_fp32=True)
    torch.cuda.synchronize()
    # Hk = HV here: v-head h reads q head h
    dh_ref, dh0_ref = oracle.state_grad_scan(inp.q[:, :, heads], do[:, :, heads], inp.scale,
                                             g=inp.g[:, :, heads], dht=dht[:, heads], split_size=64)
    check("dh", dh.cpu()[:, heads], dh_ref, torch.bfloat16, rel=STATE_SCAN_REL)
    check("dh0", dh0.cpu()[:, heads], dh0_ref, torch.bfloat16, rel=STATE_SCAN_REL)


@pytest.mark.parametrize("gate", ["gamma+gv", "kda"])
def test_bwd_dh_split_of_three_chunks(gate):
    """split_size = 192 (a stored gradient every third chunk), odd lengths, GQA."""
    inp = workloads.make_prefill(1, 455, 1, 2, 64, 64, dtype=torch.bfloat16, seed=79, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=[390, 0, 65], name="bwd_split192")
    _case(inp, gate, 192, seed=80)


@pytest.mark.parametrize("gate", ["gdn", "kda", "gamma+gv", "gv"])
def test_bwd_dh_grouped_query_heads(gate):
    """The page's grouped form of chunk_bwd_kernel_dh: HQ = 4 query / output
    heads (q and dO per query head, one dh each) read the gates of head
    i_hq // NG, NG = 2 (Hk = HV = 4, 2 gate heads)."""
    inp = workloads.make_prefill(1, 290, 4, 4, 64, 64, dtype=torch.bfloat16, seed=83,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=[100, 190], name="bwd_grouped")
    _case(inp, gate, 64, seed=84, fp32_states=True, gate_heads=2)


def test_bwd_dh_b4_t4096_bf16_states_sampled_heads():
    """The bench shape with the page's default storage (bf16 dh)."""
    inp = workloads.gdn_bf16_b4_t4096()
    B, T, Hk, HV, K, V = inp.dims
    rng = np.random.default_rng(85)
    heads = [2, 14]
    do = torch.from_numpy(rng.standard_normal((B, T, HV, V)).astype(np.float32)).to(torch.bfloat16)
    dht = torch.from_numpy((rng.standard_normal((B, HV, V, K)) * 0.1).astype(np.float32))
    print(f"bwd dh full size bf16 states heads={heads}", flush=True)
    dh, dh0 = binding.chunk_bwd_dh(dv(inp.q), dv(do), g=dv(inp.g), scale=inp.scale, dht=dv(dht), split_size=64)
    torch.cuda.synchronize()
    assert dh.dtype == torch.bfloat16
    dh_ref, dh0_ref = oracle.state_grad_scan(inp.q[:, :, heads], do[:, :, heads], inp.scale,
                                             g=inp.g[:, :, heads], dht=dht[:, heads], split_size=64)
    check("dh", dh.cpu()[:, heads], dh_ref, torch.bfloat16)
    check("dh0", dh0.cpu()[:, heads], dh0_ref, torch.bfloat16, rel=STATE_SCAN_REL)


# the scalar-gate kernel's ring of four LDS slots (loads three chunks ahead)
# and its loop unrolled by four: sequences of 0, 1, 2, ..., 8, 9 and 10 chunks
# with ragged tails, both key widths, bf16 and fp32 stored states
RING_LENS = [0, 1, 65, 130, 255, 320, 384, 448, 512, 513, 577]


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("S,fp32_states", [(64, False), (128, True)])
@pytest.mark.parametrize("gate", ["gdn", "gamma"])
def test_bwd_dh_ring_chunk_counts(K, S, fp32_states, gate):
    inp = workloads.make_prefill(1, sum(RING_LENS), 2, 4, K, K, dtype=torch.bfloat16, seed=90 + K, h0=True,
                                 seqlens=RING_LENS, name="bwd_dh_ring")
    _case(inp, gate, S, seed=91, fp32_states=fp32_states)
