"""GPU test of the no-allocation prefill entry point (gdn_chunk_fwd_noalloc,
C ABI): its outputs equal gdn_chunk_fwd's (same kernels, so bit for bit) and
meet the parity bar against the oracle, on two calls in a row, the second
smaller; a call beyond the scratch size is refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_61_amd import binding, workloads
from tests.tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
dv = lambda t: None if t is None else t.to(DEV)


def _both(inp, split=None):
    B, T, Hk, HV, K, V = inp.dims
    N = inp.num_seqs
    cu = dv(inp.cu_seqlens)
    # the existing entry point, with its own workspace
    res = binding.gdn_chunk_fwd(dv(inp.q), dv(inp.k), dv(inp.v), dv(inp.g), dv(inp.beta), scale=inp.scale,
                                h0=dv(inp.h0), cu_seqlens=cu, split_size=split, states_in_fp32=True,
                                cu_seqlens_cpu=inp.cu_seqlens)
    # the no-allocation entry point, every output preallocated, called through ctypes
    o = torch.empty((B, T, HV, V), dtype=inp.q.dtype, device=DEV)
    ht = torch.empty((N, HV, V, K), dtype=torch.float32, device=DEV)
    hs = None if split is None else torch.empty_like(res[2])
    q, k, v, g, beta, h0 = (dv(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0))
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = binding.lib().gdn_chunk_fwd_noalloc(
        p(q), p(k), p(v), p(g), None, p(beta), ctypes.c_float(inp.scale), p(h0), p(ht), p(hs), split or 0,
        0 if hs is None else hs.shape[0], binding.GDN_DTYPE_F32, p(cu), N, B, T, Hk, HV, K, V, 64,
        binding.GDN_DTYPE_BF16 if inp.q.dtype == torch.bfloat16 else binding.GDN_DTYPE_F32,
        p(o), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, binding.lib().gdn_last_error()
    torch.cuda.synchronize()
    return res, (o, ht, hs)


@pytest.mark.parametrize("first,second", [
    ((2, 300, 2, 4, 128, None), (1, 100, 1, 2, 128, None)),
    ((1, 500, 2, 4, 128, [200, 1, 299]), (1, 130, 2, 4, 64, [64, 66])),
])
def test_noalloc_matches_chunk_fwd_twice(first, second):
    for n, (B, T, Hk, HV, K, lens) in enumerate((first, second)):
        print(f"no-alloc call {n}: B={B} T={T} Hk={Hk} HV={HV} K={K} lens={lens}", flush=True)
        inp = workloads.make_prefill(B, T, Hk, HV, K, K, dtype=torch.bfloat16, seed=200 + 7 * n + T, h0=True,
                                     seqlens=lens, name=f"noalloc{n}")
        ref, got = _both(inp, split=64 if n == 0 else None)
        assert torch.equal(got[0], ref[0]), "o differs from gdn_chunk_fwd"
        assert torch.equal(got[1], ref[1]), "ht differs from gdn_chunk_fwd"
        if n == 0:
            assert torch.equal(got[2], ref[2]), "snapshots differ from gdn_chunk_fwd"
        o_ref, ht_ref = oracle.gdn_recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, h0=inp.h0,
                                             cu_seqlens=inp.cu_seqlens)
        check("o", got[0].cpu(), o_ref, torch.bfloat16)
        check("ht", got[1].cpu(), ht_ref, torch.bfloat16)


def test_noalloc_refuses_oversized_call():
    cap = binding.noalloc_max_bytes()
    assert cap == 96 << 20
    L = binding.lib()
    # B=1 T=2^20 HV=4 K=V=128 bf16 needs about 1.1 GB of workspace: refused on the host
    need = binding.workspace_bytes(1, 1 << 20, 4, 4, 128, 128, 1, torch.bfloat16)
    assert need > cap
    fake = ctypes.c_void_p(1 << 20)
    st = L.gdn_chunk_fwd_noalloc(fake, fake, fake, None, None, fake, ctypes.c_float(1.0), None, None, None, 0, 0, 0,
                                 None, 0, 1, 1 << 20, 4, 4, 128, 128, 64, binding.GDN_DTYPE_BF16, fake, None)
    assert st == 2 and b"no-allocation" in L.gdn_last_error()
