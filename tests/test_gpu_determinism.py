"""Run-to-run determinism on the GPU, through the C ABI.

No value depends on the order in which work-groups run (there are no atomics
and no reductions across work-groups), so every entry point called twice on
the same inputs must return bitwise-identical results.  The prefill must also
not depend on what its workspace held before the call: every workspace byte
it reads was written earlier in the same call, so a workspace filled with
0xFF bytes (NaN as fp32, -1 as int32) gives the same bits as a zeroed one."""

import pytest
import torch

from gated_delta_rule_61_amd import binding, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
d = lambda t: None if t is None else t.to(DEV)


def _bits(t):
    """A tensor's raw bits (NaN-safe equality)."""
    if t is None:
        return None
    t = t.contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(a, b, what):
    assert len(a) == len(b)
    for i, (x, y) in enumerate(zip(a, b)):
        if x is None:
            assert y is None
            continue
        assert torch.equal(_bits(x), _bits(y)), f"{what}: output {i} differs"


def _workspaces(nbytes):
    return (torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV),
            torch.zeros((nbytes,), dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("case", ["gdn_dense", "gdn_varlen_gqa_snapshots", "gdn_gamma_fp32", "kda_varlen",
                                  "gdn_64_column"])
def test_prefill_bitwise_repeatable_and_workspace_independent(case):
    print(f"determinism {case}", flush=True)
    kda = case.startswith("kda")
    if case == "gdn_dense":
        inp = workloads.make_prefill(2, 1000, 2, 2, 128, 128, dtype=torch.bfloat16, seed=401, h0=True)
    elif case == "gdn_varlen_gqa_snapshots":
        inp = workloads.make_prefill(1, 900, 2, 8, 128, 128, dtype=torch.bfloat16, seed=402, h0=True,
                                     seqlens=[300, 0, 1, 535, 64])
    elif case == "gdn_64_column":   # more 32-column work-groups than CUs
        inp = workloads.make_prefill(3, 300, 16, 32, 128, 128, dtype=torch.bfloat16, seed=405, h0=True)
    elif case == "gdn_gamma_fp32":
        inp = workloads.make_prefill(2, 300, 1, 2, 64, 64, dtype=torch.float32, seed=403, gate="none", h0=True)
    else:
        inp = workloads.make_prefill(1, 700, 2, 2, 128, 128, dtype=torch.bfloat16, seed=404, gate="kda",
                                     h0=True, seqlens=[129, 571])
    B, T, Hk, HV, K, V = inp.dims
    nbytes = binding.workspace_bytes(B, T, Hk, HV, K, V, inp.num_seqs, inp.q.dtype, kda=kda)
    snap = 128 if case == "gdn_varlen_gqa_snapshots" else None
    gamma = torch.full((HV,), -0.03, dtype=torch.float32) if case == "gdn_gamma_fp32" else None

    def run(ws):
        if kda:
            r = binding.kda_chunk_fwd(d(inp.q), d(inp.k), d(inp.v), d(inp.gk), d(inp.beta), scale=inp.scale,
                                      h0=d(inp.h0), cu_seqlens=d(inp.cu_seqlens), workspace=ws)
        else:
            r = binding.gdn_chunk_fwd(d(inp.q), d(inp.k), d(inp.v), d(inp.g), d(inp.beta), scale=inp.scale,
                                      h0=d(inp.h0), cu_seqlens=d(inp.cu_seqlens), workspace=ws, split_size=snap,
                                      g_gamma=d(gamma), cu_seqlens_cpu=inp.cu_seqlens)
        torch.cuda.synchronize()
        return [None if x is None else x.clone() for x in r]

    ff, zero = _workspaces(nbytes)
    first = run(ff)
    _same(first, run(zero), f"{case}: 0xFF against zeroed workspace")
    _same(first, run(ff), f"{case}: second call")
    for x in first:
        if x is not None:
            assert bool(torch.isfinite(x.float()).all()), f"{case}: non-finite output"


@pytest.mark.parametrize("T", [1, 2, 4])
def test_decode_bitwise_repeatable(T):
    print(f"determinism decode T={T}", flush=True)
    dec = workloads.make_decode(37, T, 4, 8, 128, 128, seed=410 + T, pool=50,
                                indices=list(range(49, 12, -1)))
    outs = []
    for _ in range(2):
        state = dec.state.to(DEV).clone()
        o = binding.gdn_decode(d(dec.q), d(dec.k), d(dec.v), d(dec.a), d(dec.b), d(dec.A_log), d(dec.dt_bias),
                               state, d(dec.indices), scale=dec.scale)
        torch.cuda.synchronize()
        outs.append([o.clone(), state])
    _same(outs[0], outs[1], f"decode T={T}")


@pytest.mark.parametrize("gate", ["gdn", "kda", "gv"])
def test_state_scans_bitwise_repeatable(gate):
    print(f"determinism state scans gate={gate}", flush=True)
    inp = workloads.make_prefill(1, 500, 2, 4, 128, 128, dtype=torch.bfloat16, seed=420, h0=True,
                                 gate="kda" if gate == "kda" else "gdn", seqlens=[250, 250])
    gv = None
    if gate == "gv":
        gv = -torch.rand((1, 500, 4, 128), generator=torch.Generator().manual_seed(421)) * 0.05
    kw = dict(g=d(inp.g) if gate != "kda" else None, gk=d(inp.gk), gv=d(gv), cu_seqlens=d(inp.cu_seqlens),
              split_size=64, cu_seqlens_cpu=inp.cu_seqlens)
    do = torch.randn((1, 500, 4, 128), generator=torch.Generator().manual_seed(422)).to(torch.bfloat16)
    runs = []
    for _ in range(2):
        h, ht = binding.chunk_fwd_h(d(inp.k), d(inp.v), h0=d(inp.h0), **kw)
        dh, dh0 = binding.chunk_bwd_dh(d(inp.q), d(do), scale=inp.scale, dht=d(inp.h0), **kw)
        torch.cuda.synchronize()
        runs.append([h, ht, dh, dh0])
    _same(runs[0], runs[1], f"state scans gate={gate}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_chunk_intra_bitwise_repeatable_and_workspace_independent(dtype):
    print(f"determinism chunk_intra {dtype}", flush=True)
    inp = workloads.make_prefill(1, 900, 2, 4, 128, 128, dtype=dtype, seed=430, seqlens=[300, 0, 1, 535, 64])
    nbytes = binding.lib().gdn_chunk_intra_workspace_bytes(inp.num_seqs)

    def run(ws):
        r = binding.gdn_chunk_intra(d(inp.k), d(inp.v), d(inp.g), d(inp.beta), cu_seqlens=d(inp.cu_seqlens),
                                    workspace=ws)
        torch.cuda.synchronize()
        return [x.clone() for x in r]

    ff, zero = _workspaces(nbytes)
    first = run(ff)
    _same(first, run(zero), "chunk_intra: 0xFF against zeroed workspace")
    _same(first, run(ff), "chunk_intra: second call")
