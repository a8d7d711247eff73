"""Build libpa.so (the HIP kernels and the C entry points) for gfx950, in-tree.

    python -m paged_kv_attention_table_amd.build

Each .hip source is compiled to an object in parallel, then linked into
paged_kv_attention_table_amd/libpa.so.  Flags: -O3, no fast-math (the merge relies
on IEEE infinities), and packed-fp32 instructions disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    noise = [ln for ln in (proc.stderr or "").splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, 16))) as ex:
        objects = list(ex.map(_compile, sources))
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objects, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY} from {len(sources)} sources")
    return LIBRARY


if __name__ == "__main__":
    build()
