#!/usr/bin/env python3
"""Throughput of the gated-delta-rule hot path on one MI355X.

One step = one ``gdn_chunk_fwd`` call (gate cumsum, intra-chunk solve, chunk
scan fused with the output) over the GDN workload B=4 T=4096 H=16 K=V=128,
bf16 q/k/v, fp32 gate/beta/state, zero h0, final state stored; inputs are
seeded synthetic tensors already resident in HBM.  ``value`` is prefill
tokens/s (B*T per call).  The same JSON line carries the other workloads --
the varlen GQA prefill (8 packed sequences, Hk=16, HV=32, h0 in), the KDA
prefill (B=2 T=8192 H=32), the decode step (B=256 HV=32 K=V=128 bf16 state,
T=1 and T=4), the prefill -> decode handoff, the prefill with state
snapshots, the backward and forward state scans -- each with its roofline,
and the fp64 CPU oracle timed on all host cores, per workload.

Roofline figures use the method's own bytes and FLOPs (not this
implementation's intermediates):
  * bytes: q and k once per key head, v and o once, g (GDN) or gk (KDA) and
    beta once, KDA's Aqk / Akk_inv outputs, the fp32 initial (when given) and
    final states;
  * FLOPs per token per v-head: 6 dk dv + 80 (3 dk + 2 dv) + 2048 (the
    block-lower K K^T, Q K^T, w, u, Aqk Vn products, w h, K^T Vn, Q h, and the
    block merge of a 64-token chunk).
``roofline.achieved`` is the method's bytes per call over the average
duration of the dominant kernel (library HIP events on the launch stream,
inside the timed loop); ``roofline.call`` the same bytes over the whole call.

Every timing starts with ~0.25 s of untimed back-to-back calls of the same
step (``clock_settle_s``: the GPU clock ramps over the first ~30 ms of a
burst), then the W warm-up calls, then the K timed calls.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
NUM_SIMDS = 1024                 # 256 CUs x 4 SIMDs


def method_flops_per_token(dk: int, dv: int) -> int:
    """Algorithmic FLOPs per token per v-head of the chunked prefill (C = 64,
    16-token sub-blocks): the block-lower products the method computes, not
    the dense 64 x 64 work it skips."""
    return 6 * dk * dv + 80 * (3 * dk + 2 * dv) + 2048


def method_bytes_prefill(inp, kda: bool, io: int = 2) -> int:
    """Minimum HBM bytes of one prefill call (see the module docstring)."""
    B, T, Hk, HV, K, V = inp.dims
    tok = B * T
    N = inp.num_seqs
    b = 2 * tok * Hk * K * io + 2 * tok * HV * V * io + tok * HV * 4   # q, k; v, o; beta
    if kda:
        b += tok * HV * K * 4 + 2 * tok * HV * 64 * io                  # gk; Aqk, Akk_inv out
    else:
        b += tok * HV * 4                                               # g
    b += N * HV * V * K * 4                                             # ht
    if inp.h0 is not None:
        b += N * HV * V * K * 4                                         # h0
    return b


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--skip-extra", action="store_true", help="prefill workload only")
    p.add_argument("--only", choices=["prefill", "decode", "kda", "varlen", "handoff", "bwd_dh", "fwd_h", "intra_wu",
                                      "copy",
                                      "cpu", "snapshots"],
                   default=None,
                   help="run one workload (for profiling) and print its figures")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-cache prefill timing")
    p.add_argument("--decode-batch", type=int, default=256, help="batch of --only decode")
    p.add_argument("--states", choices=["both", "bf16", "fp32"], default="both",
                   help="stored-state dtypes of the state-scan workloads")
    return p.parse_args()


CLOCK_SETTLE_S = 0.25


def settle(fn, seconds=CLOCK_SETTLE_S):
    """Untimed back-to-back calls for `seconds`: the GPU clock ramps up over
    the first tens of milliseconds of a burst of work (the prefill call takes
    ~20 % longer during the first ~30 ms), and every timing here is of the
    steady state."""
    import torch
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        n += 8
    return n


def timed(fn, steps, warmup):
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def graph_ms_per_call(torch, step, replays, per=8):
    """Milliseconds per call when `per` back-to-back calls are captured in a
    HIP graph and the graph is replayed: the launch cost a serving loop pays
    once per replay instead of once per call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per):
            step()
    settle(g.replay)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(replays):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / (replays * per)


def stage_times(binding, torch, step, steps):
    """Average duration of each library stage over `steps` calls: HIP events
    recorded by the library on the launch stream around every kernel."""
    binding.profile_read()
    binding.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = binding.profile_read()
    binding.profile_enable(False)
    return {s: prof[s][0] / prof[s][1] for s in prof if prof[s][1]}


# --------------------------------------------------------------- counters
def source_hash() -> str:
    """Hash of the kernel sources and their compiler flags (the same hash the
    profile summaries record), taken over the code only: comments,
    indentation and blank lines are dropped, so that an edit of the text
    around a kernel does not void its measured counters."""
    import glob
    import hashlib
    import re
    from gated_delta_rule_61_amd import build
    h = hashlib.sha256()
    h.update(repr((build.HIPCC_FLAGS, sorted(build.FILE_FLAGS.items()))).encode())
    for f in sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_61_amd", "csrc", "*"))):
        with open(f, encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        lines = (re.sub(r"//.*", "", ln).strip() for ln in text.splitlines())
        h.update(os.path.basename(f).encode())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def _profile_json(name: str):
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            d = json.load(f)
    except OSError:
        return None
    return d if d.get("source_sha") == source_hash() else None


def measured_traffic(key: str):
    """HBM bytes per launch of one kernel from the committed rocprofv3 byte
    counters, or None when the kernels changed since they were taken."""
    d = _profile_json("hbm_traffic.json")
    if d is None or key not in d.get("per_launch", {}):
        return None
    t = d["per_launch"][key]
    return int(t["fetch_bytes"] + t["write_bytes"])


def mfma_counters(key: str):
    """MFMA counters per launch of one kernel from the committed rocprofv3
    run (MFMA-busy fraction of the SIMDs over the kernel's active cycles and
    the MFMA FLOPs it executed), or None when the kernels changed since."""
    d = _profile_json("mfma_counters.json")
    if d is None or key not in d.get("per_launch", {}):
        return None
    return d["per_launch"][key]


def roofline(kernel, kernel_ms, call_ms, mbytes, mflops, meas_key):
    """Roofline of the dominant kernel on the method's bytes; the call on the
    same bytes; the method's FLOPs as a fraction of the bf16 MFMA peak."""
    dur = kernel_ms * 1e-3
    meas = measured_traffic(meas_key)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    roof = {"kernel": kernel, "bound": "hbm" if mflops / mbytes < ridge else "mfma",
            "achieved": round(mbytes / dur / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None if meas is None else round(meas / dur / 1e9, 1)
    roof["kernel_ms"] = round(kernel_ms, 5)
    roof["method_bytes"] = mbytes
    roof["method_flops"] = mflops
    roof["measured_bytes"] = meas
    roof["call"] = {"ms": round(call_ms, 5), "achieved_GBps": round(mbytes / (call_ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(mbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "mfma_frac_method_flops": round(mflops / (call_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "roofline_ceiling_mfma_frac": round(min(1.0, mflops / mbytes / ridge), 4),
                    # achieved FLOP/s over the attainable min(MFMA peak, HBM peak x intensity)
                    "roofline_frac": round(mflops / (call_ms * 1e-3)
                                           / min(MFMA_BF16_PEAK_TFLOPS * 1e12, HBM_PEAK_GBS * 1e9 * mflops / mbytes), 4)}
    return roof


# --------------------------------------------------------------- workloads
def bench_prefill(args, binding, workloads, torch):
    """B=4 T=4096 H=16 K=V=128 bf16 GDN prefill: the headline."""
    inp = workloads.gdn_bf16_b4_t4096()
    dev = "cuda:0"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    g, beta = inp.g.to(dev), inp.beta.to(dev)
    B, T, Hk, HV, K, V = inp.dims
    o = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.workspace_bytes(B, T, Hk, HV, K, V, B, torch.bfloat16),
                     dtype=torch.uint8, device=dev)

    def step():
        binding.gdn_chunk_fwd(q, k, v, g, beta, scale=inp.scale, out=o, workspace=ws)

    ms = timed(step, args.steps, args.warmup)
    st = stage_times(binding, torch, step, args.steps)
    # cold-cache variant: 1 GiB scratch written between calls, only the call timed
    cold = []
    scratch = None if args.no_cold else torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(0 if args.no_cold else min(args.steps, 10)):
        scratch.fill_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del scratch
    tokens = B * T
    mbytes = method_bytes_prefill(inp, kda=False)
    mflops = method_flops_per_token(K, V) * tokens * HV
    dom = max(("intra", "scan"), key=lambda s: st.get(s, 0.0))
    return {"ms": ms, "tokens": tokens, "stage_ms": st,
            "roofline": roofline(dom, st[dom], ms, mbytes, mflops, f"prefill:{dom}"),
            "mfma_counters": {s: mfma_counters(f"prefill:{s}") for s in ("intra", "scan")},
            "cold_ms": sorted(cold)[len(cold) // 2] if cold else None}


def bench_varlen(args, binding, workloads, torch):
    """GDN varlen + GQA: 8 packed sequences, h0 in, ht out (the largest GDN
    workload)."""
    inp = workloads.gdn_varlen_gqa()
    dev = "cuda:0"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    g, beta, h0 = inp.g.to(dev), inp.beta.to(dev), inp.h0.to(dev)
    cu = inp.cu_seqlens.to(dev)
    B, T, Hk, HV, K, V = inp.dims
    N = inp.num_seqs
    o = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.workspace_bytes(B, T, Hk, HV, K, V, N, torch.bfloat16),
                     dtype=torch.uint8, device=dev)

    def step():
        binding.gdn_chunk_fwd(q, k, v, g, beta, scale=inp.scale, h0=h0, cu_seqlens=cu, out=o,
                              workspace=ws)

    ms = timed(step, max(args.steps // 2, 1), 1)
    st = stage_times(binding, torch, step, max(args.steps // 2, 1))
    mbytes = method_bytes_prefill(inp, kda=False)
    mflops = method_flops_per_token(K, V) * T * HV
    lens = (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1]).tolist()
    return {"workload": f"gdn_chunk_fwd varlen {N} seqs (lengths {lens}), T={T}, Hk={Hk} HV={HV} "
                        f"K=V={K} bf16, h0 in, ht out",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "mfma_frac_method_flops": round(mflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kernels_ms": {s: round(v, 5) for s, v in st.items()},
            "roofline": roofline("scan", st["scan"], ms, mbytes, mflops, "varlen:scan"),
            "mfma_counters": {s: mfma_counters(f"varlen:{s}") for s in ("intra", "scan")}}


def bench_kda(args, binding, workloads, torch):
    """KDA B=2 T=8192 H=32 K=V=128 bf16, Aqk / Akk_inv returned."""
    inp = workloads.kda_bf16_b2_t8192()
    dev = "cuda:0"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    gk, beta = inp.gk.to(dev), inp.beta.to(dev)
    B, T, Hk, HV, K, V = inp.dims
    ws = torch.empty(binding.workspace_bytes(B, T, Hk, HV, K, V, B, torch.bfloat16, kda=True),
                     dtype=torch.uint8, device=dev)

    def step():
        binding.kda_chunk_fwd(q, k, v, gk, beta, scale=inp.scale, workspace=ws)

    ms = timed(step, max(args.steps // 2, 1), 1)
    st = stage_times(binding, torch, step, max(args.steps // 2, 1))
    mbytes = method_bytes_prefill(inp, kda=True)
    mflops = method_flops_per_token(K, V) * B * T * HV
    dom = max(("intra", "scan"), key=lambda s: st.get(s, 0.0))
    return {"workload": f"kda_chunk_fwd B={B} T={T} H={HV} K=V={K} bf16, Aqk and Akk_inv out",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "mfma_frac_method_flops": round(mflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kernels_ms": {s: round(v, 5) for s, v in st.items()},
            "roofline": roofline(dom, st[dom], ms, mbytes, mflops, f"kda:{dom}"),
            "mfma_counters": {s: mfma_counters(f"kda:{s}") for s in ("intra", "scan")}}


def bench_decode(args, binding, workloads, torch, T, B=256):
    inp = (workloads.decode_b256(T) if B == 256 else
           workloads.make_decode(B, T, 16, 32, 128, 128, seed=1004, name=f"decode_b{B}"))
    dev = "cuda:0"
    t = {n: getattr(inp, n).to(dev) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")}
    state = inp.state.to(dev)
    B, _, H, K = inp.q.shape
    HV, V = inp.v.shape[2], inp.v.shape[3]
    o = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=dev)

    def step():
        binding.gdn_decode(t["q"], t["k"], t["v"], t["a"], t["b"], t["A_log"], t["dt_bias"], state,
                           scale=inp.scale, out=o)

    ms = timed(step, args.steps, args.warmup)
    kms = stage_times(binding, torch, step, args.steps)["decode"]
    gms = graph_ms_per_call(torch, step, max(args.steps, 4))
    state_bytes = 2 * B * HV * V * K * 2
    other = (2 * B * T * H * K + 2 * B * T * HV * V + 2 * B * T * HV) * 2 + 2 * HV * 4
    # One kernel per call: the back-to-back loop time per call bounds the
    # kernel's duration from above (it adds only the launch gaps).  Events
    # around every single launch (kernel_ms_bracketed) stretch this short,
    # write-heavy kernel by 10-15 %, so the rates use the loop time.
    meas = measured_traffic(f"decode:T{T}" if B == 256 else f"decode_b{B}:T{T}")
    return {
        "workload": f"gdn_decode B={B} T={T} H={H} HV={HV} K=V={K} bf16 state",
        "ms_per_call": round(ms, 5),
        "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "state_GBps": round(state_bytes / (ms * 1e-3) / 1e9, 1),
        "total_GBps": round((state_bytes + other) / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round((state_bytes + other) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_ms_bracketed": round(kms, 5),
        "graph_ms_per_call": round(gms, 5),
        "graph_tokens_per_s": round(B * T / (gms * 1e-3), 1),
        "method_bytes": state_bytes + other,
        "measured_bytes": meas,
        "traffic_GBps": None if meas is None else round(meas / (ms * 1e-3) / 1e9, 1),
    }


def bench_snapshots(args, binding, workloads, torch, base_ms):
    """The headline prefill with state snapshots every 64 tokens (every chunk,
    the densest setting) and every 1024 tokens, stored in bf16 (the state-scan
    page's default, states in the input dtype) and in fp32."""
    inp = workloads.gdn_bf16_b4_t4096()
    dev = "cuda:0"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    g, beta = inp.g.to(dev), inp.beta.to(dev)
    B, T, Hk, HV, K, V = inp.dims
    o = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.workspace_bytes(B, T, Hk, HV, K, V, B, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    res = {}
    for S in (64, 1024):
        for fp32 in (False, True):
            dt = torch.float32 if fp32 else torch.bfloat16
            hs = torch.empty((binding.snapshot_count(B, T, S), HV, V, K), dtype=dt, device=dev)

            def step():
                binding.gdn_chunk_fwd(q, k, v, g, beta, scale=inp.scale, out=o, workspace=ws,
                                      split_size=S, h_snap=hs, states_in_fp32=fp32)

            ms = timed(step, max(args.steps // 2, 1), 1)
            st = stage_times(binding, torch, step, max(args.steps // 2, 1))
            res[f"split{S}_{'fp32' if fp32 else 'bf16'}"] = {
                "ms_per_call": round(ms, 5), "overhead_vs_no_snapshots": round(ms / base_ms - 1, 4),
                "kernels_ms": {k: round(v, 5) for k, v in st.items()},
                "snapshot_MB": round(hs.numel() * hs.element_size() / 1e6, 1)}
            del hs
    return res


def _state_scan(args, binding, torch, make_step, stage, nbytes_of, desc):
    out = {"workload": desc}
    for fp32 in {"both": (False, True), "bf16": (False,), "fp32": (True,)}[args.states]:
        step = make_step(fp32)
        ms = timed(step, max(args.steps // 2, 1), 1)
        kms = stage_times(binding, torch, step, max(args.steps // 2, 1))[stage]
        nbytes = nbytes_of(4 if fp32 else 2)
        meas = measured_traffic(f"{stage}:{'fp32' if fp32 else 'bf16'}")
        out["fp32_states" if fp32 else "bf16_states"] = {
            "ms_per_call": round(ms, 5), "kernel_ms": round(kms, 5),
            "GBps": round(nbytes / (kms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "measured_bytes": meas}
    return out


def bench_bwd_dh(args, binding, workloads, torch):
    """Backward state-gradient scan on the headline shape (B=4 T=4096 H=16
    K=V=128, bf16 q / dout, scalar gate), dh every chunk (bf16 and fp32),
    dht in, dh0 out."""
    inp = workloads.gdn_bf16_b4_t4096()
    dev = "cuda:0"
    B, T, Hk, HV, K, V = inp.dims
    gen = torch.Generator(device=dev)
    gen.manual_seed(1006)
    q, g = inp.q.to(dev), inp.g.to(dev)
    do = torch.randn((B, T, HV, V), generator=gen, device=dev).to(torch.bfloat16)
    dht = torch.randn((B, HV, V, K), generator=gen, device=dev) * 0.1

    def make_step(fp32):
        return lambda: binding.chunk_bwd_dh(q, do, g=g, scale=inp.scale, dht=dht, split_size=64,
                                            states_in_fp32=fp32)

    nchunks = B * ((T + 63) // 64)
    nbytes = lambda sb: (B * T * Hk * K * 2 + B * T * HV * V * 2 + B * T * HV * 4
                         + nchunks * HV * V * K * sb + 2 * B * HV * V * K * 4)
    return _state_scan(args, binding, torch, make_step, "bwd_dh", nbytes,
                       f"gdn_chunk_bwd_dh B={B} T={T} H={HV} K=V={K} bf16, dh every 64 tokens, dht in, dh0 out")


def bench_fwd_h(args, binding, workloads, torch):
    """Forward decay-only state scan on the headline shape (B=4 T=4096 H=16
    K=V=128, bf16 k / v, scalar gate), h at every chunk (bf16 and fp32), ht
    out."""
    inp = workloads.gdn_bf16_b4_t4096()
    dev = "cuda:0"
    B, T, Hk, HV, K, V = inp.dims
    k, v, g = inp.k.to(dev), inp.v.to(dev), inp.g.to(dev)

    def make_step(fp32):
        return lambda: binding.chunk_fwd_h(k, v, g=g, split_size=64, states_in_fp32=fp32)

    nchunks = B * ((T + 63) // 64)
    nbytes = lambda sb: (B * T * Hk * K * 2 + B * T * HV * V * 2 + B * T * HV * 4
                         + nchunks * HV * V * K * sb + B * HV * V * K * 4)
    return _state_scan(args, binding, torch, make_step, "fwd_h", nbytes,
                       f"gdn_chunk_fwd_h B={B} T={T} H={HV} K=V={K} bf16, h every 64 tokens, ht out")


def bench_handoff(args, binding, workloads, torch):
    """Prefill -> decode handoff: 256 sequences' fp32 final states (32 heads,
    K = V = 128) into a shuffled 256-slot bf16 pool."""
    dev = "cuda:0"
    N, HV, K, V = 256, 32, 128, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(1005)
    ht = torch.randn((N, HV, V, K), generator=gen, device=dev) * 0.1
    pool = torch.zeros((N, HV, V, K), dtype=torch.bfloat16, device=dev)
    idx = torch.randperm(N, generator=gen, device=dev).to(torch.int32)

    def step():
        binding.state_to_pool(ht, pool, idx)

    ms = timed(step, args.steps, args.warmup)
    nbytes = N * HV * V * K * (4 + 2)
    return {"workload": f"gdn_state_to_pool N={N} HV={HV} K=V={K}, fp32 -> bf16, shuffled slots",
            "ms_per_call": round(ms, 5), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "measured_bytes": measured_traffic("handoff")}


def bench_intra_wu(args, binding, workloads, torch):
    """The intra-chunk step on its own (gdn_chunk_intra: A, w and u) on the
    headline shape.  Bytes per token and v-head: k (shared by the HV / Hk
    v-heads of a q / k head), v, g and beta in; A, w and u out."""
    inp = workloads.gdn_bf16_b4_t4096()
    dev = "cuda:0"
    k, v, g, beta = inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev)
    B, T, Hk, HV, K, V = inp.dims

    def step():
        binding.gdn_chunk_intra(k, v, g, beta)

    ms = timed(step, args.steps, args.warmup)
    nbytes = B * T * (Hk * K * 2 + HV * (V * 2 + 4 + 4 + 64 * 2 + K * 2 + V * 2))
    return {"workload": f"gdn_chunk_intra B={B} T={T} H={HV} K=V={K} bf16, A, w and u out",
            "ms_per_call": round(ms, 5), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
            "measured_bytes": measured_traffic("intra_wu")}


# --------------------------------------------------------------- CPU oracle
_CPU = {}   # workload inputs, set before the worker processes fork


def _oracle_prefill_head(task):
    """The oracle on one v-head of a prefill workload (heads are independent):
    the head's slices of the inputs, the oracle as it stands."""
    import oracle
    name, j = task
    inp = _CPU[name]
    B, T, Hk, HV, K, V = inp.dims
    jk = j // (HV // Hk)
    hs = slice(jk, jk + 1)
    vs = slice(j, j + 1)
    h0 = None if inp.h0 is None else inp.h0[:, vs]
    if inp.gk is not None:
        oracle.kda_recurrent(inp.q[:, :, hs], inp.k[:, :, hs], inp.v[:, :, vs], inp.gk[:, :, vs], inp.beta[:, :, vs],
                             inp.scale, h0=h0, cu_seqlens=inp.cu_seqlens)
        oracle.chunk_intra_matrices(inp.q[:, :, hs], inp.k[:, :, hs], inp.beta[:, :, vs], inp.scale,
                                    gk=inp.gk[:, :, vs], cu_seqlens=inp.cu_seqlens)
    else:
        oracle.gdn_recurrent(inp.q[:, :, hs], inp.k[:, :, hs], inp.v[:, :, vs], inp.g[:, :, vs], inp.beta[:, :, vs],
                             inp.scale, h0=h0, cu_seqlens=inp.cu_seqlens)
    return j


def _oracle_decode_rows(task):
    """The decode oracle on a block of batch rows (rows are independent)."""
    import oracle
    name, r0, r1 = task
    inp = _CPU[name]
    sl = slice(r0, r1)
    oracle.gdn_decode(inp.q[sl], inp.k[sl], inp.v[sl], inp.a[sl], inp.b[sl], inp.A_log, inp.dt_bias,
                      inp.state[sl], scale=inp.scale)
    return r0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class _Host:
    """A workload's inputs as host numpy arrays (bf16 values widened exactly
    to fp32), so that the forked workers never call into torch."""

    def __init__(self, inp):
        for name, val in vars(inp).items():
            if hasattr(val, "detach"):
                val = val.detach().cpu()
                val = (val.float() if val.is_floating_point() else val).numpy()
            setattr(self, name, val)
        self.dims = getattr(inp, "dims", None)
        self.num_seqs = getattr(inp, "num_seqs", None)


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def cpu_baselines(workloads):
    """The fp64 oracle timed on every host core (one worker process per core,
    work split over independent (sequence, v-head) recurrences or decode batch
    rows), per workload: whole workloads, no sampling.  Runs before the GPU
    is initialised (the workers are forked)."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    _CPU["prefill"] = _Host(workloads.gdn_bf16_b4_t4096())
    _CPU["varlen"] = _Host(workloads.gdn_varlen_gqa())
    _CPU["kda"] = _Host(workloads.kda_bf16_b2_t8192())
    _CPU["decode_T1"] = _Host(workloads.decode_b256(1))
    _CPU["decode_T4"] = _Host(workloads.decode_b256(4))
    out = {"cores": cores, "cpu": cpu_model(), "kind": "oracle"}
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_worker_init) as pool:
        for name in ("prefill", "varlen", "kda"):
            inp = _CPU[name]
            B, T, Hk, HV, K, V = inp.dims
            t0 = time.perf_counter()
            pool.map(_oracle_prefill_head, [(name, j) for j in range(HV)], chunksize=1)
            dt = time.perf_counter() - t0
            out[name] = {"seconds": round(dt, 2), "tokens_per_s": round(B * T / dt, 1),
                         "sample": f"whole workload ({B * T} tokens x {HV} v-heads)"
                                   + (", plus the Aqk / Akk_inv matrices" if name == "kda" else "")}
        for T in (1, 4):
            name = f"decode_T{T}"
            inp = _CPU[name]
            B = inp.q.shape[0]
            step = max(1, B // cores)
            t0 = time.perf_counter()
            pool.map(_oracle_decode_rows, [(name, r, min(r + step, B)) for r in range(0, B, step)], chunksize=1)
            dt = time.perf_counter() - t0
            out[name] = {"seconds": round(dt, 2), "tokens_per_s": round(B * T / dt, 1),
                         "sample": f"one whole call ({B} rows x {T} tokens x 32 v-heads)"}
    _CPU.clear()
    return out


# --------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the method shards over "
              "(sequence, head) with no communication between GPUs", file=sys.stderr)
        sys.exit(2)
    from gated_delta_rule_61_amd import workloads
    cpu = None
    if args.only == "cpu" or (args.only is None and not args.no_cpu_baseline):
        cpu = cpu_baselines(workloads)   # before anything touches the GPU
        if args.only == "cpu":
            print(json.dumps({"cpu_oracle": cpu}), flush=True)
            return
    import torch
    from gated_delta_rule_61_amd import binding
    binding.lib()
    assert torch.cuda.is_available(), "needs a GPU"

    if args.only == "decode":
        B = args.decode_batch
        print(json.dumps({"decode": {"T1": bench_decode(args, binding, workloads, torch, 1, B),
                                     "T4": bench_decode(args, binding, workloads, torch, 4, B)}}), flush=True)
        return
    if args.only == "copy":
        # calibration for the HBM byte counters: a plain 512 MiB device copy
        src = torch.ones(1 << 27, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "calls": args.steps}), flush=True)
        return
    single = {"kda": bench_kda, "bwd_dh": bench_bwd_dh, "fwd_h": bench_fwd_h, "handoff": bench_handoff,
              "varlen": bench_varlen, "intra_wu": bench_intra_wu}
    if args.only in single:
        print(json.dumps({args.only: single[args.only](args, binding, workloads, torch)}), flush=True)
        return

    pf = bench_prefill(args, binding, workloads, torch)
    ms = pf["ms"]
    if args.only == "snapshots":
        print(json.dumps({"prefill_ms": ms, "kernels_ms": pf["stage_ms"],
                          "snapshots": bench_snapshots(args, binding, workloads, torch, ms)}), flush=True)
        return
    tokens = pf["tokens"]
    roof = pf["roofline"]
    out = {
        "metric": "prefill tokens/s + % MFMA peak; decode tokens/s + state HBM GB/s (1 GPU)",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gdn_chunk_fwd B=4 T=4096 H=16 K=V=128 BT=64, bf16 q/k/v, fp32 g/beta/state, "
                               "zero h0, ht stored",
                   "global_batch": 4, "seq_len": 4096},
        "clock_settle_s": CLOCK_SETTLE_S,
        "mfma_frac_method_flops": roof["call"]["mfma_frac_method_flops"],
        "cold_ms_per_step": None if pf["cold_ms"] is None else round(pf["cold_ms"], 5),
        "kernels_ms": {s: round(v, 5) for s, v in pf["stage_ms"].items()},
        "roofline": roof,
        "mfma_counters": pf["mfma_counters"],
    }
    if not args.skip_extra and args.only is None:
        out["varlen"] = bench_varlen(args, binding, workloads, torch)
        try:
            out["kda"] = bench_kda(args, binding, workloads, torch)
        except Exception as e:  # the KDA path reports its own status
            out["kda"] = {"error": f"{type(e).__name__}: {e}"}
        out["decode"] = {"T1": bench_decode(args, binding, workloads, torch, 1),
                         "T4": bench_decode(args, binding, workloads, torch, 4)}
        # small batches are latency-bound: the kernel's own duration
        # (kernel_ms_bracketed) is the figure; the loop rate is launch-bound
        out["decode_b1"] = {"T1": bench_decode(args, binding, workloads, torch, 1, 1),
                            "T4": bench_decode(args, binding, workloads, torch, 4, 1)}
        out["handoff"] = bench_handoff(args, binding, workloads, torch)
        out["snapshots"] = bench_snapshots(args, binding, workloads, torch, ms)
        out["bwd_dh"] = bench_bwd_dh(args, binding, workloads, torch)
        out["fwd_h"] = bench_fwd_h(args, binding, workloads, torch)
        out["intra_wu"] = bench_intra_wu(args, binding, workloads, torch)
    if cpu is not None:
        c = cpu["prefill"]
        out["cpu_baseline"] = {"value": c["tokens_per_s"], "unit": "tokens/s", "cores": cpu["cores"],
                               "kind": "oracle",
                               "sample": f"{c['sample']}, {c['seconds']} s on {cpu['cores']} cores of "
                                         f"{cpu['cpu']}: numpy fp64 token-by-token recurrence, one worker "
                                         f"process per core over the v-heads"}
        out["cpu_oracle"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
