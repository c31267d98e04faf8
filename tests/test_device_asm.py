"""Checks on the library's own gfx950 device assembly (CPU only: compiled here
with the build's flags, nothing is run).

The direct-to-LDS loads are inline assembly that set M0 (the LDS address of
such a load) and issue the load right after.  M0 is a reserved register: a
clobber list cannot make the compiler preserve it around the statement, so the
kernels are correct only while compiler-generated code keeps no value of its
own in M0.  This test compiles every source to device assembly and checks that
each M0 access is an `s_mov_b32 m0, ...` followed directly by a
`buffer_load_* ... lds` -- the pairs the inline assembly emits."""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from linear_cross_entropy_tiled_amd import build

SOURCES = [s for s in build.SOURCES if s != "flce_api.hip"]   # the API file holds no device code


def _device_asm(src, tmp):
    out = os.path.join(tmp, src + ".s")
    cmd = [build.hipcc(), *build.HIPCC_FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode(errors="replace")[-2000:]
    return open(out).read()


def test_m0_is_only_set_for_direct_to_lds_loads():
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, tmp), SOURCES))
    pairs = 0
    for src, text in zip(SOURCES, texts):
        lines = [l.split(";")[0].strip() for l in text.splitlines()]
        lines = [l for l in lines if l and not l.startswith((".", "//"))]
        for i, l in enumerate(lines):
            if not re.search(r"\bm0\b", l):
                continue
            assert l.startswith("s_mov_b32 m0,"), f"{src}: compiler-generated M0 access: {l!r}"
            nxt = lines[i + 1] if i + 1 < len(lines) else ""
            assert re.match(r"buffer_load_dword\S* .* lds$", nxt), f"{src}: M0 set without its load: {l!r} / {nxt!r}"
            pairs += 1
    assert pairs > 0
