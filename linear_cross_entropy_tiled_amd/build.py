"""Builds libflce.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m linear_cross_entropy_tiled_amd.build [--verbose] [--host-sanitizers]

The library is built in-tree, next to this file, so that it travels with the
source tree.  Every call recompiles.

--host-sanitizers builds libflce_hostsan.so instead: the same sources with the
host code (argument validation, planning, launch set-up) compiled under
AddressSanitizer and UndefinedBehaviorSanitizer (-Xarch_host, so the device
code is built as usual).  It is for host-side tests only: load it with
FLCE_LIB_PATH pointing at it and the compiler's shared ASan runtime in
LD_PRELOAD (``sanitizer_runtime()``); tests/test_abi_host_sanitized.py does
that for the C-ABI validation tests.
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
SOURCES = ["flce_api.hip", "flce_forward.hip", "flce_backward.hip", "flce_chunked.hip", "flce_fused.hip",
           "flce_noalloc.hip"]
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


SAN_LIB_PATH = os.path.join(PKG_DIR, "libflce_hostsan.so")
HOST_SANITIZER_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload into a host process)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       stderr=subprocess.DEVNULL)
    path = r.stdout.decode().strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not hits:
            raise RuntimeError("the shared ASan runtime (libclang_rt.asan-x86_64.so) was not found")
        path = hits[0]
    return path


def build_host_sanitized(verbose: bool = False) -> str:
    """libflce_hostsan.so: host code under ASan + UBSan, linked against the shared ASan runtime."""
    return build(verbose, extra_flags=HOST_SANITIZER_FLAGS, out_path=SAN_LIB_PATH,
                 link_flags=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                             "-shared-libasan"], opt="-O1")


def build(verbose: bool = False, extra_flags=None, out_path: str = LIB_PATH, link_flags=None, opt: str = "-O3") -> str:
    cc = hipcc()
    flags = [f if f != "-O3" else opt for f in HIPCC_FLAGS] + list(extra_flags or [])
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
        tmp_lib = out_path + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(link_flags or []), *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            print(r.stdout.decode(errors="replace"), file=sys.stderr)
            raise RuntimeError("linking libflce.so failed")
        os.replace(tmp_lib, out_path)
    return out_path


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv:
        print(build_host_sanitized(verbose="--verbose" in sys.argv))
    else:
        print(build(verbose="--verbose" in sys.argv))
