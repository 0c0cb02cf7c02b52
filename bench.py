#!/usr/bin/env python3
"""Throughput of the gated-delta-rule hot path on one MI355X.

One step = one ``gdn_chunk_fwd`` call (gate cumsum, intra-chunk solve, chunk
scan fused with the output) over the GDN workload B=4 T=4096 H=16 K=V=128,
bf16 q/k/v, fp32 gate/beta/state, zero h0, final state stored; inputs are
seeded synthetic tensors already resident in HBM.  ``value`` is prefill
tokens/s (B*T per call).  The same JSON line also carries the decode step
(B=256, HV=32, K=V=128, bf16 state, T=1 and T=4: tokens/s and state GB/s),
the varlen GQA prefill (8 packed sequences, Hk=16, HV=32, h0 in), the KDA
prefill (B=2 T=8192 H=32), the prefill -> decode state handoff (256 states
into a bf16 pool), the prefill with state snapshots, the backward state-gradient
scan, the per-kernel roofline of the
dominant prefill kernel (live HIP-event timing inside the library, on the
launch stream) and the fp64 CPU oracle timed on a bounded sample.

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

# Algorithmic FLOPs per token per v-head of each prefill kernel (dk = dv = d):
#   intra: block-lower K K^T and Q K^T (2 x 80 d; 10 of 16 16x16 blocks of a
#          64-token chunk) + the 16 block-merge products (16 * 2 * 16^3 / 64)
#   scan:  K S^T, Q S^T, K^T Vn (3 x 2 d^2) + block-lower Ainv R and Aqk Vn (2 x 80 d)
def intra_flops_per_token(d: int) -> int:
    return 2 * 80 * d + 16 * 2 * 16 ** 3 // 64


def scan_flops_per_token(d: int) -> int:
    return 6 * d * d + 2 * 80 * d


# Algorithmic HBM bytes per launch (bf16 io: 2-byte q/k/v/o; Ainv and Aqk
# staged as fp16 64-wide rows; gate factors as 4 fp32 planes; fp32 state):
#   intra: reads q, k (per k-head), g, beta; writes Ainv, Aqk, gate factors
#   scan:  reads q, k, v, Ainv, Aqk, gate factors (and h0); writes o, ht
def intra_bytes(B, T, Hk, HV, K, V, io=2):
    return 2 * B * T * Hk * K * io + 2 * B * T * HV * 4 + 2 * B * T * HV * 64 * 2 + B * T * HV * 16


def scan_bytes(B, T, Hk, HV, K, V, N, io=2, h0=False):
    state = N * HV * K * V * 4
    return (2 * B * T * Hk * K * io + B * T * HV * V * io + 2 * B * T * HV * 64 * 2 + B * T * HV * 16
            + B * T * HV * V * io + state * (2 if h0 else 1))


# The headline "% MFMA" uses the method's algorithmic count per token per
# v-head, 6 dk dv + 80 (3 dk + 2 dv) + 2048 (block-lower K K^T, Q K^T, w, u,
# Aqk Vn, w h, K^T Vn, Q h and the merge).
def method_flops_per_token(dk: int, dv: int) -> int:
    return 6 * dk * dv + 80 * (3 * dk + 2 * dv) + 2048


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=16384)
    p.add_argument("--skip-extra", action="store_true", help="prefill workload only")
    p.add_argument("--only", choices=["prefill", "decode", "kda", "varlen", "handoff", "bwd_dh", "fwd_h", "copy"],
                   default=None,
                   help="run one workload (for profiling) and print its figures")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-cache prefill timing")
    p.add_argument("--decode-batch", type=int, default=256, help="batch of --only decode")
    return p.parse_args()


def timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall


def bench_prefill(args, binding, workloads, torch):
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

    ms, wall = timed(step, args.steps, args.warmup)
    # live per-kernel timing: library events on the launch stream, same timed loop
    binding.profile_read()
    binding.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = binding.profile_read()
    binding.profile_enable(False)
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
    return dict(inp=inp, ms=ms, wall=wall, prof=prof, tokens=tokens, HV=HV, K=K, V=V,
                cold_ms=sorted(cold)[len(cold) // 2] if cold else None)


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

    ms, _ = timed(step, args.steps, args.warmup)
    binding.profile_read()
    binding.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = binding.profile_read()
    binding.profile_enable(False)
    kms = prof["decode"][0] / max(prof["decode"][1], 1)
    state_bytes = 2 * B * HV * V * K * 2
    other = (2 * B * T * H * K + 2 * B * T * HV * V + 2 * B * T * HV) * 2 + 2 * HV * 4
    # One kernel per call: the back-to-back loop time per call bounds the
    # kernel's duration from above (it adds only the launch gaps).  Events
    # around every single launch (kernel_ms_bracketed) stretch this short,
    # write-heavy kernel by 10-15 %, so the rates use the loop time.
    return {
        "workload": f"gdn_decode B={B} T={T} H={H} HV={HV} K=V={K} bf16 state",
        "ms_per_call": round(ms, 5),
        "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "state_GBps": round(state_bytes / (ms * 1e-3) / 1e9, 1),
        "total_GBps": round((state_bytes + other) / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round((state_bytes + other) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_ms_bracketed": round(kms, 5),
        "measured_bytes": measured_traffic(f"decode:T{T}" if B == 256 else f"decode_b{B}:T{T}"),
    }


def bench_kda(args, binding, workloads, torch):
    inp = workloads.kda_bf16_b2_t8192()
    dev = "cuda:0"
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    gk, beta = inp.gk.to(dev), inp.beta.to(dev)
    B, T, Hk, HV, K, V = inp.dims
    ws = torch.empty(binding.workspace_bytes(B, T, Hk, HV, K, V, B, torch.bfloat16, kda=True),
                     dtype=torch.uint8, device=dev)

    def step():
        binding.kda_chunk_fwd(q, k, v, gk, beta, scale=inp.scale, workspace=ws)

    ms, _ = timed(step, max(args.steps // 2, 1), 1)
    flops = method_flops_per_token(K, V) * B * T * HV
    return {"workload": f"kda_chunk_fwd B={B} T={T} H={HV} K=V={K} bf16",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "mfma_frac_method_flops": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def bench_varlen(args, binding, workloads, torch):
    """GDN varlen + GQA: 8 packed sequences, h0 in, ht out."""
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

    ms, _ = timed(step, max(args.steps // 2, 1), 1)
    binding.profile_read()
    binding.profile_enable(True)
    for _ in range(max(args.steps // 2, 1)):
        step()
    torch.cuda.synchronize()
    prof = binding.profile_read()
    binding.profile_enable(False)
    stage_ms = {s: prof[s][0] / prof[s][1] for s in prof if prof[s][1]}
    flops = method_flops_per_token(K, V) * T * HV
    sb = scan_bytes(B, T, Hk, HV, K, V, N, h0=True)
    lens = (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1]).tolist()
    return {"workload": f"gdn_chunk_fwd varlen {N} seqs (lengths {lens}), T={T}, Hk={Hk} HV={HV} "
                        f"K=V={K} bf16, h0 in, ht out",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "mfma_frac_method_flops": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kernels_ms": {s: round(v, 5) for s, v in stage_ms.items()},
            "scan_hbm_frac": round(sb / (stage_ms["scan"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            if stage_ms.get("scan") else None,
            "scan_measured_bytes": measured_traffic("varlen:scan")}


def bench_snapshots(args, binding, workloads, torch, base_ms):
    """The headline prefill with fp32 state snapshots every 64 tokens (every
    chunk, the densest setting) and every 1024 tokens."""
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
        hs = torch.empty((binding.snapshot_count(B, T, S), HV, V, K), dtype=torch.float32, device=dev)

        def step():
            binding.gdn_chunk_fwd(q, k, v, g, beta, scale=inp.scale, out=o, workspace=ws,
                                  split_size=S, h_snap=hs, states_in_fp32=True)

        ms, _ = timed(step, max(args.steps // 2, 1), 1)
        res[f"split{S}"] = {"ms_per_call": round(ms, 5), "overhead_vs_no_snapshots": round(ms / base_ms - 1, 4),
                            "snapshot_MB": round(hs.numel() * 4 / 1e6, 1)}
        del hs
    return res


def bench_bwd_dh(args, binding, workloads, torch):
    """Backward state-gradient scan on the headline shape (B=4 T=4096 H=16
    K=V=128, bf16 q / dout, scalar gate), dh every chunk, dht in, dh0 out."""
    inp = workloads.gdn_bf16_b4_t4096()
    dev = "cuda:0"
    B, T, Hk, HV, K, V = inp.dims
    gen = torch.Generator(device=dev)
    gen.manual_seed(1006)
    q, g = inp.q.to(dev), inp.g.to(dev)
    do = torch.randn((B, T, HV, V), generator=gen, device=dev).to(torch.bfloat16)
    dht = torch.randn((B, HV, V, K), generator=gen, device=dev) * 0.1

    def step():
        binding.chunk_bwd_dh(q, do, g=g, scale=inp.scale, dht=dht, split_size=64, states_in_fp32=True)

    nchunks = B * ((T + 63) // 64)
    nbytes = (B * T * Hk * K * 2 + B * T * HV * V * 2 + B * T * HV * 4
              + nchunks * HV * V * K * 4 + 2 * B * HV * V * K * 4)
    return _bench_state_scan(args, binding, torch, step, "bwd_dh", nbytes,
                             f"gdn_chunk_bwd_dh B={B} T={T} H={HV} K=V={K} bf16, dh every 64 tokens, dht in, dh0 out")


def bench_fwd_h(args, binding, workloads, torch):
    """Forward decay-only state scan on the headline shape (B=4 T=4096 H=16
    K=V=128, bf16 k / v, scalar gate), h at every chunk, ht out."""
    inp = workloads.gdn_bf16_b4_t4096()
    dev = "cuda:0"
    B, T, Hk, HV, K, V = inp.dims
    k, v, g = inp.k.to(dev), inp.v.to(dev), inp.g.to(dev)

    def step():
        binding.chunk_fwd_h(k, v, g=g, split_size=64, states_in_fp32=True)

    nchunks = B * ((T + 63) // 64)
    nbytes = (B * T * Hk * K * 2 + B * T * HV * V * 2 + B * T * HV * 4
              + nchunks * HV * V * K * 4 + B * HV * V * K * 4)
    return _bench_state_scan(args, binding, torch, step, "fwd_h", nbytes,
                             f"gdn_chunk_fwd_h B={B} T={T} H={HV} K=V={K} bf16, h every 64 tokens, ht out")


def _bench_state_scan(args, binding, torch, step, stage, nbytes, desc):
    ms, _ = timed(step, max(args.steps // 2, 1), 1)
    binding.profile_read()
    binding.profile_enable(True)
    for _ in range(max(args.steps // 2, 1)):
        step()
    torch.cuda.synchronize()
    prof = binding.profile_read()
    binding.profile_enable(False)
    kms = prof[stage][0] / max(prof[stage][1], 1)
    return {"workload": desc,
            "ms_per_call": round(ms, 5), "kernel_ms": round(kms, 5),
            "GBps": round(nbytes / (kms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "measured_bytes": measured_traffic(stage)}


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

    ms, _ = timed(step, args.steps, args.warmup)
    nbytes = N * HV * V * K * (4 + 2)
    return {"workload": f"gdn_state_to_pool N={N} HV={HV} K=V={K}, fp32 -> bf16, shuffled slots",
            "ms_per_call": round(ms, 5), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes, "measured_bytes": measured_traffic("handoff")}


def source_hash() -> str:
    """Hash of the kernel sources (the same hash the profile summaries record)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_61_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch of one kernel from the committed rocprofv3 byte
    counters, or None when the kernels changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except OSError:
        return None
    if d.get("source_sha") != source_hash() or key not in d.get("per_launch", {}):
        return None
    t = d["per_launch"][key]
    return int(t["fetch_bytes"] + t["write_bytes"])


def cpu_baseline(args, workloads):
    """fp64 oracle on a bounded sample of the same prefill workload."""
    import oracle
    inp = workloads.gdn_bf16_b4_t4096()
    B, T = inp.q.shape[:2]
    S = min(args.cpu_sample_tokens, B * T)
    rows = max(1, S // T)
    toks = min(S, T) if rows == 1 else T
    t0 = time.perf_counter()
    oracle.gdn_recurrent(inp.q[:rows, :toks], inp.k[:rows, :toks], inp.v[:rows, :toks],
                         inp.g[:rows, :toks], inp.beta[:rows, :toks], inp.scale)
    dt = time.perf_counter() - t0
    n = rows * toks
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"batch rows 0..{rows - 1}, tokens 0..{toks - 1} ({n} of {B * T} tokens, all 16 heads), "
                      f"{dt:.1f} s; numpy fp64 token-by-token recurrence, single thread"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the method shards over "
              "(sequence, head) with no communication, see DESIGN.md", file=sys.stderr)
        sys.exit(2)
    import torch
    from gated_delta_rule_61_amd import binding, workloads
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
    if args.only == "kda":
        print(json.dumps({"kda": bench_kda(args, binding, workloads, torch)}), flush=True)
        return
    if args.only == "bwd_dh":
        print(json.dumps({"bwd_dh": bench_bwd_dh(args, binding, workloads, torch)}), flush=True)
        return
    if args.only == "fwd_h":
        print(json.dumps({"fwd_h": bench_fwd_h(args, binding, workloads, torch)}), flush=True)
        return
    if args.only == "handoff":
        print(json.dumps({"handoff": bench_handoff(args, binding, workloads, torch)}), flush=True)
        return
    if args.only == "varlen":
        print(json.dumps({"varlen": bench_varlen(args, binding, workloads, torch)}), flush=True)
        return
    pf = bench_prefill(args, binding, workloads, torch)
    ms = pf["ms"]
    tokens = pf["tokens"]
    HV, K, V = pf["HV"], pf["K"], pf["V"]
    prof = pf["prof"]
    stage_ms = {s: (prof[s][0] / prof[s][1] if prof[s][1] else 0.0) for s in ("intra", "scan")}
    flops = {"intra": intra_flops_per_token(K) * tokens * HV, "scan": scan_flops_per_token(K) * tokens * HV}
    B, T, Hk = pf["inp"].dims[:3]
    nbytes = {"intra": intra_bytes(B, T, Hk, HV, K, V), "scan": scan_bytes(B, T, Hk, HV, K, V, B)}
    dom = max(stage_ms, key=stage_ms.get)
    # roofline bound of the dominant kernel: arithmetic intensity vs the ridge
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    dur = stage_ms[dom] * 1e-3
    meas = measured_traffic(f"prefill:{dom}")
    if flops[dom] / nbytes[dom] >= ridge:
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(flops[dom] / dur / 1e12, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(nbytes[dom] / dur / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None if meas is None else round(meas / dur / 1e9, 1)
    roof["algorithmic_bytes"] = nbytes[dom]
    roof["algorithmic_flops"] = flops[dom]
    roof["measured_bytes"] = meas
    method = method_flops_per_token(K, V) * tokens * HV
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
        "config": {"workload": "gdn_chunk_fwd B=4 T=4096 H=16 K=V=128 BT=64, bf16 q/k/v, fp32 g/beta/state, zero h0, ht stored",
                   "global_batch": 4, "seq_len": 4096},
        "mfma_frac_method_flops": round(method / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "cold_ms_per_step": None if pf["cold_ms"] is None else round(pf["cold_ms"], 5),
        "kernels_ms": {s: round(v, 5) for s, v in stage_ms.items()},
        "roofline": roof,
        "kernels_hbm_frac": {s: round(nbytes[s] / (stage_ms[s] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                             for s in stage_ms if stage_ms[s] > 0},
    }
    if not args.skip_extra and args.only is None:
        out["decode"] = {"T1": bench_decode(args, binding, workloads, torch, 1),
                         "T4": bench_decode(args, binding, workloads, torch, 4)}
        # small batches are latency-bound: the kernel's own duration
        # (kernel_ms_bracketed) is the figure; the loop rate is launch-bound
        out["decode_b1"] = {"T1": bench_decode(args, binding, workloads, torch, 1, 1),
                            "T4": bench_decode(args, binding, workloads, torch, 4, 1)}
        out["varlen"] = bench_varlen(args, binding, workloads, torch)
        out["handoff"] = bench_handoff(args, binding, workloads, torch)
        out["snapshots"] = bench_snapshots(args, binding, workloads, torch, ms)
        out["bwd_dh"] = bench_bwd_dh(args, binding, workloads, torch)
        out["fwd_h"] = bench_fwd_h(args, binding, workloads, torch)
        try:
            out["kda"] = bench_kda(args, binding, workloads, torch)
        except Exception as e:  # KDA path reports its own status
            out["kda"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_cpu_baseline and args.only is None:
        out["cpu_baseline"] = cpu_baseline(args, workloads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
