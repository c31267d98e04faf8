"""Builds libflce.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m linear_cross_entropy_tiled_amd.build [--verbose]

The library is built in-tree, next to this file, so that it travels with the
source tree.  Every call recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libflce.so")
SOURCES = ["flce_api.hip", "flce_forward.hip", "flce_backward.hip", "flce_chunked.hip", "flce_fused.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libflce.so)")


def build(verbose: bool = False, extra_flags=None) -> str:
    cc = hipcc()
    flags = HIPCC_FLAGS + list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="flce_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, pr in procs:
            out, _ = pr.communicate()
            text = out.decode(errors="replace")
            # the host pass does not know the packed-fp32 feature; that note is expected
            text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
            if pr.returncode != 0:
                failed.append(src)
                print(text, file=sys.stderr)
            elif verbose and text.strip():
                print(text)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB_PATH + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            print(r.stdout.decode(errors="replace"), file=sys.stderr)
            raise RuntimeError("linking libflce.so failed")
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
