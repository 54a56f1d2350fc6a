"""Build libbased.so (the gfx950 HIP library) in-tree with hipcc.

    python -m linear_attention_sequence_taylor_amd.build [--jobs N]

Each source under csrc/ is compiled to an object in _build/ (parallel), then
linked into linear_attention_sequence_taylor_amd/libbased.so.  Always
recompiles: a build is the check that every kernel compiles for gfx950.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "libbased")
LIB_PATH = os.path.join(PKG, "libbased.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code (the compiler
# would otherwise fuse pairs of fp32 ops into v_pk_* instructions).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
                "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
# Per-source extras.  The backward kernels keep MFMA results in ordinary
# VGPRs (their scores and products feed vector code right away; with AGPR
# results every value would be copied out first), and are scheduled for
# instruction-level parallelism (the chunked form ran 4% shorter, with
# bit-identical results).  prefill_mfma_ilp.hip holds the prefill
# instances that run faster under the iterative form of that scheduler.
SOURCE_FLAGS = {
    "prefill_backward_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "prefill_mfma_ilp.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbased.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, os.cpu_count() or 1, len(sources))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(sources)} sources")
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    build(ap.parse_args().jobs)
