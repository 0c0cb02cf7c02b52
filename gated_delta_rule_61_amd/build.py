"""Build the gfx950 shared library ``libgdn61.so`` in-tree with hipcc.

    python -m gated_delta_rule_61_amd.build

Every HIP source under ``csrc/`` is compiled for gfx950 only (in parallel,
into a temporary directory) and the objects are linked into one shared
object next to this file.  Packed-fp32 instruction forms are disabled for the
device code.  A few sources take extra code-generation flags (``FILE_FLAGS``).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgdn61.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-munsafe-fp-atomics",
]

# The bf16 scan and the decode kernels keep MFMA accumulators in ordinary
# VGPRs, which their VALU work reads and writes right away; with the
# accumulation registers the compiler copies them back and forth.  The state
# scans and the KDA intra kernel run about 3 % faster under the compiler's
# ILP-first scheduler (same occupancy; the intra kernel spills 8 bytes per
# lane instead of 12).
FILE_FLAGS = {
    "chunk_scan_gdn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "state_scans.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "kda_intra.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}

NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd: list, verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    return msgs


def build(verbose: bool = False, extra: list | None = None) -> str:
    srcs = sources()
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="gdn61_build_") as tmpd:
        jobs = []
        for src in srcs:
            obj = os.path.join(tmpd, os.path.basename(src) + ".o")
            flags = FILE_FLAGS.get(os.path.basename(src), [])
            jobs.append(([hipcc(), *HIPCC_FLAGS, *inc, *flags, *(extra or []), "-c", src, "-o", obj], obj))
        workers = min(len(jobs), os.cpu_count() or 4, 8)
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            outs = list(ex.map(lambda j: _run(j[0], verbose), jobs))
        tmp = LIB + ".tmp"
        outs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
                          *[o for _, o in jobs], "-o", tmp], verbose))
    if verbose:
        for m in outs:
            if m.strip():
                print(m)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
