"""Build the gfx950 shared library ``libgptq_mi355x.so`` in-tree with hipcc.

Run as ``python -m post_weight_quantization_04_amd.build``.  Every HIP source
under ``csrc/`` is compiled for gfx950 only, with packed-fp32 instruction
selection disabled and no fast-math, then linked into one shared library
next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libgptq_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    "-Wno-unused-const-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, obj: str) -> str:
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="gptq_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            logs = list(ex.map(_compile, srcs, objs))
        if verbose:
            for s, log in zip(srcs, logs):
                if log.strip():
                    print(f"[{os.path.basename(s)}]\n{log}", file=sys.stderr)
        tmp_lib = LIB_PATH + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
