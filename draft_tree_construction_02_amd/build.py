"""Build libdartree.so (gfx950) in-tree with hipcc.

    python -m draft_tree_construction_02_amd.build

Each HIP source is compiled to an object in parallel, then linked into
``draft_tree_construction_02_amd/libdartree.so``.  Always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdartree.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["dartree.hip", "gemm.hip", "head_wide.hip", "select.hip", "pack.hip", "attention.hip",
           "sequential.hip", "verify.hip", "head_rows128.hip", "probe.hip", "build_small.hip"]
ARCH = os.environ.get("DARTREE_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (p.stdout + p.stderr).splitlines()
            if "packed-fp32-ops" not in ln]
    return p.returncode, "\n".join(msgs)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]

    def compile_one(s):
        obj = os.path.join(BUILD, s.replace(".hip", ".o"))
        rc, out = _run([cc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", obj])
        return s, obj, rc, out

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        results = list(ex.map(compile_one, srcs))
    for s, _, rc, out in results:
        if out and (verbose or rc):
            print(f"--- {s}\n{out}", file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed on {s}")
    tmp = OUT + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                    *[o for _, o, _, _ in results]])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
