#!/usr/bin/env python3
"""Turn rocprofv3 CSV output of bench.py runs into the text summaries and the
per-launch counter tables that bench.py reads (profiles/hbm_traffic.json,
profiles/mfma_counters.json).

Expected layout of the rocprofv3 output directory (``--output-format csv -o
run``, one ``-d`` per run; the commands are printed in every summary):

  <dir>/<w>_kt/run_kernel_stats.csv                   --kernel-trace --stats
  <dir>/<w>_FETCH_SIZE/run_counter_collection.csv     --pmc FETCH_SIZE
  <dir>/<w>_WRITE_SIZE/run_counter_collection.csv     --pmc WRITE_SIZE
  <dir>/<w>_MFMA/run_counter_collection.csv           --pmc <MFMA_COUNTERS> (prefill workloads)
  <dir>/copy_FETCH_SIZE, <dir>/copy_WRITE_SIZE        bench.py --only copy (byte calibration)

Byte counters are scaled so that a plain 512 MiB device copy reads as 512 MiB
each way.  MFMA counters: SQ_INSTS_VALU_MFMA_MOPS_* count MFMA work in units of
512 FLOPs; SQ_VALU_MFMA_BUSY_CYCLES sums the MFMA-busy cycles of all SIMDs;
GRBM_GUI_ACTIVE sums the active cycles of the 8 XCDs, so the busy fraction is
busy / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs).

    python3 profile_summary.py <rocprofv3 output dir>
"""

from __future__ import annotations

import csv
import functools
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE")
NUM_XCD, NUM_SIMD = 8, 1024

# workload -> (summary file, bench.py arguments, {kernel: per-launch key})
SPECS = [
    ("prefill", "gdn_chunk_fwd_B4_T4096_H16_K128_bf16", "--only prefill",
     {"gdn_scan_bf16_kernel<128,false,2>": "prefill:scan", "gdn_intra_kernel<ushort,128,half>": "prefill:intra"}),
    ("varlen", "gdn_chunk_fwd_varlen8_gqa16x32_K128_bf16", "--only varlen",
     {"gdn_scan_bf16_kernel<128,false,4>": "varlen:scan", "gdn_intra_kernel<ushort,128,half>": "varlen:intra"}),
    ("kda", "kda_chunk_fwd_B2_T8192_H32_K128_bf16", "--only kda",
     {"kda_intra_kernel<ushort,128,half>": "kda:intra", "gdn_scan_bf16_kernel<128,true,2>": "kda:scan"}),
    ("decode", "gdn_decode_B256_HV32_K128_T1_T4", "--only decode",
     {"gdn_decode_kernel<1,256>": "decode:T1", "gdn_decode_mfma_kernel<4,4>": "decode:T4"}),
    ("decode_b1", "gdn_decode_B1_HV32_K128_T1_T4", "--only decode --decode-batch 1",
     {"gdn_decode_kernel<1,64>": "decode_b1:T1", "gdn_decode_mfma_kernel<4,1>": "decode_b1:T4"}),
    ("bwd_dh_bf16", "gdn_chunk_bwd_dh_B4_T4096_H16_K128_bf16_states", "--only bwd_dh --states bf16",
     {"state_scan_ring_kernel<128,false,true>": "bwd_dh:bf16"}),
    ("bwd_dh_fp32", "gdn_chunk_bwd_dh_B4_T4096_H16_K128_fp32_states", "--only bwd_dh --states fp32",
     {"state_scan_ring_kernel<128,false,true>": "bwd_dh:fp32"}),
    ("fwd_h_bf16", "gdn_chunk_fwd_h_B4_T4096_H16_K128_bf16_states", "--only fwd_h --states bf16",
     {"state_scan_ring_kernel<128,true,true>": "fwd_h:bf16"}),
    ("fwd_h_fp32", "gdn_chunk_fwd_h_B4_T4096_H16_K128_fp32_states", "--only fwd_h --states fp32",
     {"state_scan_ring_kernel<128,true,true>": "fwd_h:fp32"}),
    ("handoff", "gdn_state_to_pool_N256_HV32_K128", "--only handoff",
     {"state_to_pool_kernel": "handoff"}),
    ("intra_wu", "gdn_chunk_intra_B4_T4096_H16_K128_bf16", "--only intra_wu",
     {"gdn_intra_wu_bf16_kernel<128,128>": "intra_wu"}),
]
MFMA_WORKLOADS = ("prefill", "varlen", "kda")


@functools.lru_cache(None)
def _demangle(n: str) -> str:
    if not n.startswith("_Z"):
        return n
    try:
        return subprocess.run(["c++filt", n], capture_output=True, text=True).stdout.strip() or n
    except OSError:
        return n


def kernel_name(raw: str):
    """Short name of one of the library's kernels (None for other kernels)."""
    n = _demangle(raw)
    if n.startswith("_Z"):  # a c++filt that does not know _Float16 (DF16_)
        m = re.search(r"_GLOBAL__N_1(\d+)", n)
        if not m:
            return None
        ln = int(m.group(1))
        base, rest = n[m.end():m.end() + ln], n[m.end() + ln:]
        targs = {"ILi128ELb0ELi2E": "<128,false,2>", "ILi128ELb0ELi4E": "<128,false,4>",
                 "ILi128ELb1ELi2E": "<128,true,2>", "ILi128ELb0E": "<128,false>", "ILi128ELb1E": "<128,true>",
                 "ItLi128E": "<ushort,128,half>", "ILi128ELi128EE": "<128,128>"}
        return base + next((v for k, v in targs.items() if rest.startswith(k)), "")
    m = re.search(r"gdn::\(anonymous namespace\)::(\w+)(<[^>]*>)?", n)
    if not m:
        return None
    t = (m.group(2) or "").replace(" ", "").replace("unsignedshort", "ushort").replace("_Float16", "half")
    return m.group(1) + t


def counters(path: str):
    """{kernel: {counter: mean value per dispatch}} from one counter CSV."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            raw = r["Kernel_Name"]
            k = "copy" if "copyBuffer" in raw else kernel_name(raw) if "gdn" in raw else None
            if k is None:
                continue
            per = acc.setdefault(k, {}).setdefault(r["Counter_Name"], {})
            d = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(per))
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    return {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def main(out_dir: str):
    import bench
    sha = bench.source_hash()
    cf = counters(f"{out_dir}/copy_FETCH_SIZE/run_counter_collection.csv")["copy"]["FETCH_SIZE"]
    cw = counters(f"{out_dir}/copy_WRITE_SIZE/run_counter_collection.csv")["copy"]["WRITE_SIZE"]
    copy_kib = 512 * 1024
    f_fetch, f_write = copy_kib / cf, copy_kib / cw
    traffic, mfma = {}, {}
    for w, fname, args, keys in SPECS:
        if not os.path.isdir(f"{out_dir}/{w}_kt"):
            print(f"skip {w}: no kernel trace")
            continue
        F = counters(f"{out_dir}/{w}_FETCH_SIZE/run_counter_collection.csv")
        W = counters(f"{out_dir}/{w}_WRITE_SIZE/run_counter_collection.csv")
        M = (counters(f"{out_dir}/{w}_MFMA/run_counter_collection.csv")
             if w in MFMA_WORKLOADS and os.path.isdir(f"{out_dir}/{w}_MFMA") else {})
        lines = []
        with open(f"{out_dir}/{w}_kt/run_kernel_stats.csv") as f:
            rows = [r for r in csv.DictReader(f) if "gdn" in r["Name"]]
        # the timed calls: each kernel's last 20 dispatches (the trace also holds
        # the untimed clock-settle calls before them)
        durs = {}
        with open(f"{out_dir}/{w}_kt/run_kernel_trace.csv") as f:
            for r in csv.DictReader(f):
                if "gdn" in r["Kernel_Name"]:
                    durs.setdefault(kernel_name(r["Kernel_Name"]), []).append(
                        (int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        for r in rows:
            k = kernel_name(r["Name"])
            last = sorted(d for _, d in sorted(durs.get(k, []))[-20:])
            avg_ns = float(last[len(last) // 2]) if last else float(r["AverageNs"])
            fb = F.get(k, {}).get("FETCH_SIZE", 0.0) * f_fetch * 1024
            wb = W.get(k, {}).get("WRITE_SIZE", 0.0) * f_write * 1024
            key = keys.get(k)
            line = (f"{k[:38]:38s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {avg_ns / 1e3:9.2f} "
                    f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {fb / 1e6:9.1f} {wb / 1e6:9.1f}")
            if key:
                traffic[key] = {"fetch_bytes": fb, "write_bytes": wb}
            if key and k in M:
                c = M[k]
                flops = 512.0 * sum(c.get(f"SQ_INSTS_VALU_MFMA_MOPS_{t}", 0.0) for t in ("BF16", "F16", "F32"))
                active = c.get("GRBM_GUI_ACTIVE", 0.0) / NUM_XCD
                busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (active * NUM_SIMD) if active else None
                mfma[key] = {"mfma_flops": flops, "mfma_busy_frac": busy,
                             "active_cycles_per_xcd": active, "avg_ns": avg_ns,
                             "clock_GHz_from_active": active / avg_ns if avg_ns else None,
                             "raw": c}
                line += f"   mfma_busy {busy:6.3f}  mfma_TFLOP {flops / 1e12:7.4f}"
            lines.append(line)
        head = [f"# rocprofv3 kernel statistics: {fname}",
                "# commands (on one MI355X, from /tmp with TMPDIR=/tmp; <repo> is the repository root):",
                f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <out>/{w}_kt -o run -- "
                f"python3 <repo>/bench.py {args} --steps 10 --warmup 2 --no-cold",
                f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/{w}_FETCH_SIZE -o run -- "
                f"python3 <repo>/bench.py {args} --steps 3 --warmup 1 --no-cold   (then WRITE_SIZE)"]
        if M:
            head.append(f"#   rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d <out>/{w}_MFMA -o run -- "
                        f"python3 <repo>/bench.py {args} --steps 3 --warmup 1 --no-cold")
        head += ["#   python3 <repo>/profile_summary.py <out>",
                 f"# HBM bytes = FETCH_SIZE x {f_fetch:.3f} + WRITE_SIZE x {f_write:.3f} (KiB x 1024); the factors "
                 "make a plain 512 MiB device copy",
                 "#   (bench.py --only copy --steps 3 under the same two counters) read as 512 MiB each way",
                 f"# kernel source hash: {sha}",
                 "# avg_us: every dispatch (with the untimed clock-settle calls); timed_us: median of the last",
                 "#   20 dispatches (the timed calls); fetch / write: HBM bytes per dispatch", "",
                 f"{'kernel':38s}  calls    avg_us  timed_us    min_us    max_us  fetch_MB  write_MB"]
        text = "\n".join(head + lines) + "\n"
        with open(os.path.join(ROOT, "profiles", f"{fname}.txt"), "w") as f:
            f.write(text)
        print(text)
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as f:
        json.dump({"source_sha": sha, "calibration": {"fetch": f_fetch, "write": f_write}, "per_launch": traffic},
                  f, indent=1)
    with open(os.path.join(ROOT, "profiles", "mfma_counters.json"), "w") as f:
        json.dump({"source_sha": sha, "counters": MFMA_COUNTERS, "per_launch": mfma}, f, indent=1)
    print(json.dumps(mfma, indent=1))


if __name__ == "__main__":
    main(sys.argv[1])
