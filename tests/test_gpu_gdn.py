"""GPU parity of the GDN chunked prefill against the fp64 oracle (C ABI)."""

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_61_amd import binding, workloads
from tests.tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(inp, output_final_state=True):
    dv = lambda t: None if t is None else t.to(DEV)
    o, ht = binding.gdn_chunk_fwd(dv(inp.q), dv(inp.k), dv(inp.v), dv(inp.g), dv(inp.beta),
                                  scale=inp.scale, h0=dv(inp.h0),
                                  output_final_state=output_final_state,
                                  cu_seqlens=dv(inp.cu_seqlens))
    torch.cuda.synchronize()
    return o.cpu(), None if ht is None else ht.cpu()


def _ref(inp, heads=None):
    return oracle.gdn_recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0,
                                cu_seqlens=inp.cu_seqlens, heads=heads)


def _compare(inp, heads=None):
    print(f"case {inp.name} dims={inp.dims} heads={heads}", flush=True)
    o, ht = _gpu(inp)
    o_ref, ht_ref = _ref(inp, heads)
    dt = inp.q.dtype
    if heads is None:
        eo = check("o", o, o_ref, dt)
        eh = check("ht", ht, ht_ref, dt)
    else:
        eo = check("o", o[:, :, heads], o_ref[:, :, heads], dt)
        eh = check("ht", ht[:, heads], ht_ref[:, heads], dt)
    print(f"  o {eo}  ht {eh}", flush=True)


def test_gdn_fp32_small_workload():
    """fp32 io, B=1 T=256 H=2 K=V=64: every output against max-abs 1e-4."""
    _compare(workloads.gdn_fp32_small())


@pytest.mark.parametrize("T", [1, 7, 16, 63, 64, 65, 200])
def test_gdn_fp32_ragged(T):
    inp = workloads.make_prefill(2, T, 1, 2, 64, 64, dtype=torch.float32, seed=T, h0=True,
                                 name=f"fp32_T{T}")
    _compare(inp)


@pytest.mark.parametrize("K", [64, 128])
def test_gdn_bf16_ragged_gqa(K):
    inp = workloads.make_prefill(2, 200, 2, 4, K, K, dtype=torch.bfloat16, seed=K, h0=True,
                                 name=f"bf16_gqa_K{K}")
    _compare(inp)


def test_gdn_fp32_k128_no_gate():
    inp = workloads.make_prefill(1, 130, 1, 1, 128, 128, dtype=torch.float32, seed=5, gate="none",
                                 h0=True, name="fp32_nogate")
    _compare(inp)


def test_gdn_strong_gate_bf16():
    inp = workloads.make_prefill(1, 192, 2, 2, 128, 128, dtype=torch.bfloat16, seed=6, g_scale=3.0,
                                 name="bf16_strong_gate")
    _compare(inp)


def test_gdn_varlen_ragged():
    lens = [1, 63, 64, 65, 0, 130, 17]
    inp = workloads.make_prefill(1, sum(lens), 2, 4, 64, 64, dtype=torch.float32, seed=7, h0=True,
                                 seqlens=lens, name="fp32_varlen")
    _compare(inp)


def test_gdn_varlen_bf16_k128():
    lens = [300, 5, 129, 64]
    inp = workloads.make_prefill(1, sum(lens), 2, 4, 128, 128, dtype=torch.bfloat16, seed=8, h0=True,
                                 seqlens=lens, name="bf16_varlen")
    _compare(inp)


@pytest.mark.parametrize("Hk,HV,lens", [(1, 4, [130, 1, 77]), (1, 8, [64, 200]), (2, 8, None)],
                         ids=["gqa4_varlen3", "gqa8_varlen2", "gqa4_dense"])
def test_gdn_bf16_wide_gqa_groups(Hk, HV, lens):
    # the bf16 scan runs the v-heads of a (sequence, q/k head) next to each other on one XCD;
    # 4 and 8 v-heads per q/k head, with unit counts that leave padding work-groups
    T = sum(lens) if lens else 150
    B = 1 if lens else 3
    inp = workloads.make_prefill(B, T, Hk, HV, 128, 128, dtype=torch.bfloat16, seed=11 + HV, h0=True,
                                 seqlens=lens, name=f"bf16_gqa{HV // Hk}")
    _compare(inp)


@pytest.mark.parametrize("B,T,Hk,HV,lens", [(3, 300, 16, 32, None), (1, 448, 24, 24, [257, 0, 1, 190]),
                                              (3, 200, 8, 32, None)],
                         ids=["gqa2_dense", "gqa1_varlen", "gqa4_dense"])
def test_gdn_bf16_64_column_work_groups(B, T, Hk, HV, lens):
    # more 32-column work-groups than CUs: the scan runs 64-column ones (four
    # state waves; the o tile in the chunk's v buffer); every head checked
    inp = workloads.make_prefill(B, T, Hk, HV, 128, 128, dtype=torch.bfloat16, seed=500 + HV + T, h0=True,
                                 seqlens=lens, name=f"bf16_64col_{Hk}x{HV}")
    _compare(inp)


def test_gdn_no_final_state_and_empty():
    inp = workloads.make_prefill(1, 70, 1, 1, 64, 64, dtype=torch.float32, seed=9)
    o, ht = _gpu(inp, output_final_state=False)
    assert ht is None
    o_ref, _ = _ref(inp)
    check("o", o, o_ref, torch.float32)
    # T = 0: the final state is h0
    e = workloads.make_prefill(2, 0, 1, 1, 64, 64, dtype=torch.float32, seed=10, h0=True)
    o, ht = _gpu(e)
    assert o.shape == (2, 0, 1, 64)
    assert torch.equal(ht, e.h0)


def test_gdn_bf16_b4_t4096_sampled_heads():
    """B=4 T=4096 H=16 K=V=128 bf16: the oracle checks two sampled heads."""
    _compare(workloads.gdn_bf16_b4_t4096(), heads=[3, 12])


def test_gdn_varlen_gqa_workload_sampled_heads():
    """8 packed sequences of U[64, 8192] tokens, Hk=16, HV=32: two sampled
    v-heads (of different q/k heads)."""
    _compare(workloads.gdn_varlen_gqa(), heads=[0, 31])
