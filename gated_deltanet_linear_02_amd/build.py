"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

Each .hip source compiles to an object in ``_build/`` (in parallel), then
they link into ``libgdn.so`` next to this file. Run as
``python -m gated_deltanet_linear_02_amd.build``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
ARCH = "gfx950"

SOURCES = ["gdn_api.hip", "gdn_decode.hip", "gdn_norm.hip", "gdn_prefill.hip", "gdn_tune.hip"]
# gdn_prefill_inst.hip is compiled once per (bf16 I/O, chunk size): the
# chunked prefill's kernels, six objects built in parallel.
INSTANCES = [("gdn_prefill_inst.hip", f"gdn_prefill_inst_b{b}_c{c}", [f"-DGDN_INST_BF16={b}", f"-DGDN_INST_CHUNK={c}"])
             for b in (1, 0) for c in (64, 32, 16)]

# Packed-fp32 VALU forms are disabled; hipcc's host pass warns that it does
# not know the feature, which is harmless.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdn.so)")


def _compile(job) -> str:
    src, stem, defs = job
    obj = os.path.join(BUILD, stem + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    work = INSTANCES + [(s, os.path.splitext(s)[0], []) for s in SOURCES]
    jobs = min(len(work), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, work))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
