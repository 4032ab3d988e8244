"""Build librlt.so in-tree with hipcc for gfx950.

    python -m recurrent_decode_step_amd.build_lib

Each source is compiled to an object in parallel (every kernel is launched
from the file that defines it, so no device linking is needed), then the
objects are linked into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/rlt_api.hip", "csrc/rlt_kernels.hip", "csrc/rlt_encoder.hip", "csrc/rlt_train.hip",
           "csrc/rlt_peaks.hip", "csrc/rlt_fused.hip"]
OUT = os.path.join(HERE, "librlt.so")
OBJ_DIR = os.path.join(HERE, "_build")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # packed fp32 arithmetic is switched off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
# hipcc's host pass warns that it does not know the device-only feature flag
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if NOISE not in ln]
    return r.returncode, msgs


def build(verbose: bool = False, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.basename(src).replace(".hip", ".o"))
        jobs.append((obj, [hipcc, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c",
                           os.path.join(HERE, src), "-o", obj]))
    if verbose:
        for _, cmd in jobs:
            print(" ".join(cmd), flush=True)
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    failed = False
    for (obj, _), (rc, msgs) in zip(jobs, results):
        if rc != 0:
            failed = True
            sys.stderr.write("\n".join(msgs) + "\n")
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = OUT + ".tmp"
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc link failed ({rc})")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
