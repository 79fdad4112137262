"""Build libdspark.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m draft_head_step_amd.build   (or call build()).
Objects go to <repo>/_build/, the library to draft_head_step_amd/libdspark.so.

The library carries a hash of the sources and flags it was built from
(dspark_source_hash()); the binding refuses to load a library whose hash
differs from the tree's, so a stale build can never stand in for the
committed source.
"""
from __future__ import annotations

import glob
import hashlib
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdspark.so")
SOURCES = ["api.hip", "markov_step.hip", "markov_pick_greedy_row.hip", "markov_pick_greedy_col.hip",
           "markov_pick_sample_row.hip", "markov_pick_sample_col.hip", "markov_pick_bias_only.hip",
           "confidence.hip", "schedule.hip", "verify.hip", "noalloc.hip", "rnn_head.hip",
           "layout.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # never let the compiler form packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_files() -> list:
    """Every file whose content goes into the library, in a fixed order."""
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                   glob.glob(os.path.join(INCLUDE, "*.h")))
    return files


def source_hash() -> str:
    """sha256 (first 32 hex digits) over the source files' names and contents and the
    compile flags."""
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(" ".join(HIPCC_FLAGS + SOURCES).encode())
    return h.hexdigest()[:32]


# Step kernels whose waits count the loads issued after a direct-to-LDS copy
# (rank 512 without a bias output, and the fused step's last-step K-split
# kernel, which never has one).  Scratch traffic would count in the same
# counter; a spill can only make such a wait stricter, but the build insists on
# none so that the counted loads are exactly the ones in the source.
COUNTED_WAIT_KERNEL = re.compile(
    r"markov_step_(?:(?:ksplit_kernelILi\d+E|kernelILi512E)\S*Lb0E|ksplit_fin_kernelILi\d+E)")


def scratch_offenders(remarks: str) -> list:
    """Kernels of the resource-usage remarks that need scratch but must not."""
    bad = []
    name = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0 and COUNTED_WAIT_KERNEL.search(name):
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libdspark.so)")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    tag = f'-DDSPARK_SOURCE_HASH="{source_hash()}"'
    for s in SOURCES:
        obj = os.path.join(OUT_DIR, s.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, tag, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s),
               "-o", obj]
        if s.startswith("markov_pick_"):
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    spills = []
    for s, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        spills += scratch_offenders(text)
        # the host pass does not know the packed-fp32 feature; that note is harmless
        lines = [l for l in text.splitlines()
                 if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(s)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    if spills:
        raise RuntimeError("step kernels with counted waits use scratch: " + "; ".join(spills))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
