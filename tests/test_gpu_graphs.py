"""The entry points under HIP graph capture (torch.cuda.CUDAGraph).

A call queues only kernel launches on the caller's stream: no allocation, no
memset and no host synchronisation.  So a captured call replays to the same
bits as the eager call on the same buffers.  Each graph is replayed several
times with eager work and host synchronisations in between; before every
replay its outputs are overwritten, and every replay is compared with an
eager reference.  The prefill graphs are also replayed after new values are
copied into their static inputs; decode graphs advance the pool in place,
one step per replay."""

import pytest
import torch

from gated_delta_rule_61_amd import binding, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
d = lambda t: None if t is None else t.to(DEV)


def _bits(t):
    t = t.contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(got, ref, what):
    for i, (x, y) in enumerate(zip(got, ref)):
        assert torch.equal(_bits(x), _bits(y)), f"{what}: output {i} differs"


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _other_work():
    """Eager work between replays: an unrelated prefill and a sync."""
    x = workloads.make_prefill(1, 200, 1, 1, 64, 64, dtype=torch.bfloat16, seed=449)
    binding.gdn_chunk_fwd(d(x.q), d(x.k), d(x.v), d(x.g), d(x.beta), scale=x.scale)
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["gdn_varlen", "kda"])
def test_prefill_graph_replays(kind):
    print(f"graph replay prefill {kind}", flush=True)
    kda = kind == "kda"
    mk = lambda seed: workloads.make_prefill(1, 700, 2, 4, 128, 128, dtype=torch.bfloat16, seed=seed,
                                             gate="kda" if kda else "gdn", h0=True, seqlens=[450, 1, 249])
    a, b = mk(440), mk(441)
    B, T, Hk, HV, K, V = a.dims
    names = ("q", "k", "v", "gk" if kda else "g", "beta", "h0")
    st = {n: d(getattr(a, n)).clone() for n in names}
    cu = d(a.cu_seqlens)
    ws = torch.empty(binding.workspace_bytes(B, T, Hk, HV, K, V, a.num_seqs, torch.bfloat16, kda=kda),
                     dtype=torch.uint8, device=DEV)
    gate = st["gk" if kda else "g"]

    def call():
        if kda:
            return binding.kda_chunk_fwd(st["q"], st["k"], st["v"], gate, st["beta"], scale=a.scale, h0=st["h0"],
                                         cu_seqlens=cu, workspace=ws)
        return binding.gdn_chunk_fwd(st["q"], st["k"], st["v"], gate, st["beta"], scale=a.scale, h0=st["h0"],
                                     cu_seqlens=cu, workspace=ws)

    def eager(src):
        for n in names:
            st[n].copy_(d(getattr(src, n)))
        r = call()
        torch.cuda.synchronize()
        return [x.clone() for x in r]

    ref_b = eager(b)
    ref_a = eager(a)                        # leaves inputs a in the static buffers
    g, outs = _capture(call)
    for rep, (src, ref) in enumerate(((a, ref_a), (a, ref_a), (b, ref_b), (a, ref_a))):
        for n in names:
            st[n].copy_(d(getattr(src, n)))
        for x in outs:
            x.fill_(7.0)                    # the replay must rewrite every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(outs, ref, f"{kind} replay {rep}")
        _other_work()


@pytest.mark.parametrize("T", [1, 4])
def test_decode_graph_replays_advance_the_pool(T):
    print(f"graph replay decode T={T}", flush=True)
    dec = workloads.make_decode(24, T, 4, 8, 128, 128, seed=450 + T, pool=30, indices=list(range(29, 5, -1)))
    args = [d(x) for x in (dec.q, dec.k, dec.v, dec.a, dec.b, dec.A_log, dec.dt_bias)]
    idx = d(dec.indices)
    # eager: three steps from the initial pool
    pool_e = d(dec.state).clone()
    steps = []
    for _ in range(3):
        o = binding.gdn_decode(*args, pool_e, idx, scale=dec.scale)
        torch.cuda.synchronize()
        steps.append((o.clone(), pool_e.clone()))
    # graph: one step captured on its own pool; its warm-up step is undone first
    pool_g = d(dec.state).clone()
    out = torch.empty_like(steps[0][0])
    g, _ = _capture(lambda: binding.gdn_decode(*args, pool_g, idx, scale=dec.scale, out=out))
    pool_g.copy_(d(dec.state))
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same((out, pool_g), steps[rep], f"decode T={T} replay {rep}")
        _other_work()


def test_state_scan_graph_replays():
    print("graph replay fwd_h / bwd_dh", flush=True)
    inp = workloads.make_prefill(2, 300, 2, 2, 128, 128, dtype=torch.bfloat16, seed=460, h0=True)
    k, v, q, gg, h0 = d(inp.k), d(inp.v), d(inp.q), d(inp.g), d(inp.h0)
    do = torch.randn((2, 300, 2, 128), generator=torch.Generator().manual_seed(461)).to(torch.bfloat16).to(DEV)

    def call():
        h, ht = binding.chunk_fwd_h(k, v, g=gg, h0=h0, split_size=128)
        dh, dh0 = binding.chunk_bwd_dh(q, do, g=gg, scale=inp.scale, dht=h0, split_size=64)
        return h, ht, dh, dh0

    ref = [x.clone() for x in call()]
    torch.cuda.synchronize()
    g, outs = _capture(call)
    for rep in range(3):
        for x in outs:
            x.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(outs, ref, f"state scans replay {rep}")
        _other_work()


def test_chunk_intra_graph_replays():
    print("graph replay chunk_intra", flush=True)
    inp = workloads.make_prefill(1, 700, 2, 4, 128, 128, dtype=torch.bfloat16, seed=470, seqlens=[450, 1, 249])
    k, v, gg, beta, cu = d(inp.k), d(inp.v), d(inp.g), d(inp.beta), d(inp.cu_seqlens)
    ws = torch.empty(binding.lib().gdn_chunk_intra_workspace_bytes(inp.num_seqs), dtype=torch.uint8, device=DEV)

    def call():
        return binding.gdn_chunk_intra(k, v, gg, beta, cu_seqlens=cu, workspace=ws)

    ref = [x.clone() for x in call()]
    torch.cuda.synchronize()
    g, outs = _capture(call)
    for rep in range(3):
        for x in outs:
            x.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(outs, ref, f"chunk_intra replay {rep}")
        _other_work()
