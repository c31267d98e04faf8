"""C-ABI checks that need no GPU: the library loads, exports every function
include/flce.h declares, sizes workspaces, and rejects bad arguments on the
host before touching the device."""
import ctypes
import os
import re

import pytest

import linear_cross_entropy_tiled_amd as flce

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "flce.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(flce.LIB_PATH):
        from linear_cross_entropy_tiled_amd import build
        build.build()
    return flce.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(flce_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(flce.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert flce.flce_version() >= 100
    assert flce.flce_status_string(flce.FLCE_ERR_WORKSPACE_TOO_SMALL) == "workspace too small"


def test_struct_layout_matches_header():
    # 4 x int64, 4 x int32, 4 x float, int64
    assert ctypes.sizeof(flce.flce_params) == 72
    assert flce.flce_params.dtype.offset == 32 and flce.flce_params.logit_scale.offset == 48
    assert flce.flce_params.vocab_chunk.offset == 64
    # two pointers, two int32
    assert ctypes.sizeof(flce.flce_launch_timer) == 24 and flce.flce_launch_timer.capacity.offset == 16


def test_vocab_chunk_sets_the_scratch(lib):
    """flce_params.vocab_chunk: the backward's logit-gradient scratch is N_pad x chunk elements;
    0 is the library's choice; negative or not a multiple of 256 is refused."""
    n, h, v = 8192, 4096, 128256
    sizes = {}
    for vc in (4096, 8192, 16384):
        p = flce.make_params(n, h, v, dtype="bf16", reduction="sum", softcap=30.0, vocab_chunk=vc)
        rc, b = _ws(p, flce.FLCE_PASS_BACKWARD)
        assert rc == 0
        sizes[vc] = b
    # chunks of at most vocab_chunk rows, balanced over the 501 vocabulary tiles: widths 4096
    # (32 chunks), 8192 (16) and 16128 (8); the scratch grows by N * 2 bytes per row of width
    assert sizes[8192] - sizes[4096] == n * (8192 - 4096) * 2
    assert sizes[16384] - sizes[8192] == n * (16128 - 8192) * 2
    for vc, code in ((-256, flce.FLCE_ERR_INVALID_ARG), (1000, flce.FLCE_ERR_UNSUPPORTED)):
        p = flce.make_params(n, h, v, vocab_chunk=vc)
        assert _ws(p, flce.FLCE_PASS_BACKWARD)[0] == code
    # a chunk wider than the vocabulary is one chunk
    p1 = flce.make_params(512, 64, 1000, vocab_chunk=1 << 20)
    p0 = flce.make_params(512, 64, 1000)
    assert _ws(p1, flce.FLCE_PASS_BACKWARD) == _ws(p0, flce.FLCE_PASS_BACKWARD)


def test_timed_entry_points_validate_the_timer(lib):
    p = flce.make_params(64, 64, 100)
    big = 1 << 30
    ev = (ctypes.c_void_p * 4)(16, 16, 16, 16)
    kinds = (ctypes.c_int32 * 2)()
    E = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    K = ctypes.cast(kinds, ctypes.POINTER(ctypes.c_int32))
    bad = [flce.flce_launch_timer(None, K, 2, 0), flce.flce_launch_timer(E, None, 2, 0),
           flce.flce_launch_timer(E, K, -1, 0), flce.flce_launch_timer(E, K, 2, 3),
           flce.flce_launch_timer(E, K, 2, -1)]
    for t in bad:
        assert lib.flce_forward_timed(ctypes.byref(p), 16, 16, None, 16, 16, 16, None, None, 16, big, None,
                                      ctypes.byref(t)) == flce.FLCE_ERR_INVALID_ARG
        assert lib.flce_backward_timed(ctypes.byref(p), 16, 16, None, 16, 16, 16, 16, 16, None, 16, big, None,
                                       ctypes.byref(t)) == flce.FLCE_ERR_INVALID_ARG
    # a valid timer does not hide the other checks
    ok = flce.flce_launch_timer(E, K, 2, 0)
    assert lib.flce_forward_timed(ctypes.byref(p), 16, 16, None, 16, 16, 16, None, None, 16, 8, None,
                                  ctypes.byref(ok)) == flce.FLCE_ERR_WORKSPACE_TOO_SMALL
    assert ok.count == 0


def _ws(p, pass_):
    out = ctypes.c_size_t(0)
    rc = flce.load().flce_workspace_size(ctypes.byref(p), pass_, ctypes.byref(out))
    return rc, out.value


def test_workspace_sizes(lib):
    p = flce.make_params(8192, 4096, 128256, dtype="bf16", reduction="sum", softcap=30.0)
    rc, fb = _ws(p, flce.FLCE_PASS_FORWARD)
    assert rc == 0 and 0 < fb < 64 << 20
    rc, bb = _ws(p, flce.FLCE_PASS_BACKWARD)
    # dlogits chunk scratch + fp32 grad_hidden accumulator + grad_bias partials:
    # O(N*H + N*Vc + V), far below the N*V bf16 logits (2.1 GB)
    assert rc == 0 and bb < 1.2e9
    p0 = flce.make_params(0, 64, 10)
    assert _ws(p0, flce.FLCE_PASS_FORWARD)[0] == 0
    assert _ws(p0, flce.FLCE_PASS_BACKWARD)[0] == 0
    assert _ws(p, 7)[0] == flce.FLCE_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value,code", [
    ("hidden", 100, flce.FLCE_ERR_UNSUPPORTED),          # H % 8 != 0
    ("hidden", 0, flce.FLCE_ERR_INVALID_ARG),
    ("vocab", 0, flce.FLCE_ERR_INVALID_ARG),
    ("n_tokens", -1, flce.FLCE_ERR_INVALID_ARG),
    ("dtype", 7, flce.FLCE_ERR_INVALID_ARG),
    ("grad_weight_dtype", 9, flce.FLCE_ERR_INVALID_ARG),
    ("reduction", 3, flce.FLCE_ERR_INVALID_ARG),
    ("flags", 16, flce.FLCE_ERR_INVALID_ARG),
    ("z_loss", -1.0, flce.FLCE_ERR_INVALID_ARG),
    ("logit_scale", float("inf"), flce.FLCE_ERR_INVALID_ARG),
])
def test_bad_params_rejected(lib, field, value, code):
    p = flce.make_params(64, 64, 100)
    setattr(p, field, value)
    assert _ws(p, flce.FLCE_PASS_FORWARD)[0] == code
    rc = lib.flce_forward(ctypes.byref(p), 16, 16, None, 16, 16, 16, None, None, 16, 1 << 30, None)
    assert rc == code


def test_fp16_and_int32_targets_accepted(lib):
    """fp16 inputs plan like bf16 (same element size); int32 targets are a flag."""
    for pass_ in (flce.FLCE_PASS_FORWARD, flce.FLCE_PASS_BACKWARD):
        pb = flce.make_params(5000, 1024, 50000, dtype="bf16", reduction="mean")
        ph = flce.make_params(5000, 1024, 50000, dtype="f16", reduction="mean", targets_int32=True)
        pg = flce.make_params(5000, 1024, 50000, dtype="f16", grad_weight_dtype="f32")
        rb, rh, rg = _ws(pb, pass_), _ws(ph, pass_), _ws(pg, pass_)
        assert rb[0] == rh[0] == rg[0] == 0
        assert rb[1] == rh[1] == rg[1] > 0
    assert flce.make_params(8, 8, 8, targets_int32=True).flags == flce.FLCE_TARGETS_INT32


def test_null_and_misaligned_pointers_rejected(lib):
    p = flce.make_params(64, 64, 100)
    big = 1 << 30
    # NULL loss / lse / workspace / weight
    assert lib.flce_forward(ctypes.byref(p), 16, 16, None, 16, None, 16, None, None, 16, big, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward(ctypes.byref(p), 16, None, None, 16, 16, 16, None, None, 16, big, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward(ctypes.byref(p), 16, 16, None, 16, 16, 16, None, None, None, big, None) == flce.FLCE_ERR_INVALID_ARG
    # hidden not 16-byte aligned
    assert lib.flce_forward(ctypes.byref(p), 18, 16, None, 16, 16, 16, None, None, 16, big, None) == flce.FLCE_ERR_UNSUPPORTED
    # workspace too small
    assert lib.flce_forward(ctypes.byref(p), 16, 16, None, 16, 16, 16, None, None, 16, 8, None) == flce.FLCE_ERR_WORKSPACE_TOO_SMALL
    # backward: grad_bias without bias, missing grad_weight
    assert lib.flce_backward(ctypes.byref(p), 16, 16, None, 16, 16, 16, 16, 16, 16, 16, big, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_backward(ctypes.byref(p), 16, 16, None, 16, 16, 16, 16, None, None, 16, big, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_backward(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 8, None) == flce.FLCE_ERR_WORKSPACE_TOO_SMALL
    assert lib.flce_get_status(None, None) == flce.FLCE_ERR_INVALID_ARG


def test_too_large_problem_rejected(lib):
    p = flce.make_params(1 << 20, 4096, 1000)       # N*H*2 bytes >= 2 GiB
    assert _ws(p, flce.FLCE_PASS_FORWARD)[0] == flce.FLCE_ERR_UNSUPPORTED


def test_hidden_size_limit_is_exact(lib):
    # N*H*esize must stay below 2^31 bytes: 262136 x 4096 bf16 is the largest multiple
    # of 8 rows that fits (2^31 - 64 KiB), 262144 rows is exactly 2^31
    for n, ok in ((262136, True), (262144, False)):
        p = flce.make_params(n, 4096, 64)
        for pass_ in (flce.FLCE_PASS_FORWARD, flce.FLCE_PASS_BACKWARD):
            rc = _ws(p, pass_)[0]
            assert (rc == flce.FLCE_OK) == ok, (n, pass_, rc)
            if not ok:
                assert rc == flce.FLCE_ERR_UNSUPPORTED


def test_chunked_params_layout_and_validation(lib):
    # 4 x int64, 4 x int32
    assert ctypes.sizeof(flce.flce_chunked_params) == 48
    assert ctypes.sizeof(flce.flce_wmse_args) == 40

    def ws(p):
        out = ctypes.c_size_t(0)
        return lib.flce_chunked_workspace_size(ctypes.byref(p), ctypes.byref(out)), out.value

    p = flce.make_chunked_params(8192, 4096, 128256, dtype="bf16")
    rc, b = ws(p)
    # one 4096-row block of bf16 logits (1.05 GB) + the fp32 grad_weight accumulator (2.1 GB)
    assert rc == 0 and 3.0e9 < b < 3.3e9
    p = flce.make_chunked_params(8192, 4096, 128256, dtype="bf16", grad_weight_accum_dtype="weight")
    rc, b2 = ws(p)
    assert rc == 0 and b2 < b - 2e9          # "weight" accumulation needs no fp32 accumulator
    for field, value, code in (("chunk_rows", 100, flce.FLCE_ERR_UNSUPPORTED),
                               ("chunk_rows", -256, flce.FLCE_ERR_INVALID_ARG),
                               ("accum_dtype", flce.FLCE_F16, flce.FLCE_ERR_INVALID_ARG),
                               ("flags", 2, flce.FLCE_ERR_INVALID_ARG),
                               ("dtype", 5, flce.FLCE_ERR_INVALID_ARG),
                               ("hidden", 12, flce.FLCE_ERR_UNSUPPORTED)):
        q = flce.make_chunked_params(512, 64, 1000)
        setattr(q, field, value)
        assert ws(q)[0] == code, field
    # missing loss function / loss pointer: rejected before any launch
    q = flce.make_chunked_params(512, 64, 1000)
    null_fn = ctypes.cast(None, flce.CHUNK_LOSS_FN)
    assert lib.flce_chunked_linear_loss(ctypes.byref(q), 16, 16, null_fn, None, 16, 16, 16, 16, 1 << 30,
                                        None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_chunked_linear_loss(ctypes.byref(q), 16, 16, flce.weighted_mse_chunk_fn(), None, None, 16, 16,
                                        16, 1 << 30, None) == flce.FLCE_ERR_INVALID_ARG
    # the built-in loss function checks its arguments on the host
    assert lib.flce_weighted_mse_chunk(None, 0, 1, 10, 16, 16, 1, 16, None) == flce.FLCE_ERR_INVALID_ARG
    assert flce.flce_status_string(flce.FLCE_ERR_CALLBACK) == "the chunk loss function reported an error"


def test_forward_backward_workspace_and_validation(lib):
    def ws(p, rows=0):
        out = ctypes.c_size_t(0)
        return lib.flce_forward_backward_workspace_size(ctypes.byref(p), rows, ctypes.byref(out)), out.value

    p = flce.make_params(8192, 4096, 128256, dtype="bf16", reduction="sum", softcap=30.0)
    rc, b = ws(p)
    # one 4096-row block of bf16 logits (1.05 GB), the fp32 grad_weight accumulator over the two
    # blocks (2.1 GB), hidden^T of a block, grad_bias partials: far below N*V + V*H*4 = 4.2 GB
    assert rc == 0 and 3.1e9 < b < 3.4e9
    rc, b1 = ws(p, 8192)                     # one block: no fp32 accumulator
    assert rc == 0 and b1 < b
    assert ws(p, 100)[0] == flce.FLCE_ERR_UNSUPPORTED
    assert ws(p, -256)[0] == flce.FLCE_ERR_UNSUPPORTED
    pf = flce.make_params(8192, 4096, 128256, dtype="bf16", grad_weight_dtype="f32")
    rc, bf = ws(pf)
    assert rc == 0 and bf < b - 2e9          # fp32 grad_weight is its own accumulator
    pw = flce.make_params(8192, 4096, 128256, dtype="bf16", reduction="sum", grad_weight_accum_dtype="weight")
    rc, bw = ws(pw)
    assert rc == 0 and bw < b - 2e9          # summed in grad_weight's dtype: no fp32 accumulator
    assert pw.flags == flce.FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT
    assert ws(flce.make_params(0, 64, 10))[0] == 0
    q = flce.make_params(64, 64, 100)
    big = 1 << 30
    args = dict(hidden=16, weight=16, bias=None, targets=16, grad_loss=16, loss=16, lse=16, nc=None, ent=None,
                gh=16, gw=16, gb=None, ws=16, wsb=big)

    def call(**kw):
        a = dict(args, **kw)
        return lib.flce_forward_backward(ctypes.byref(q), 0, a["hidden"], a["weight"], a["bias"], a["targets"],
                                         a["grad_loss"], a["loss"], a["lse"], a["nc"], a["ent"], a["gh"], a["gw"],
                                         a["gb"], a["ws"], a["wsb"], None)
    assert call(weight=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(gw=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(grad_loss=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(loss=None) == flce.FLCE_ERR_INVALID_ARG
    assert call(gb=16) == flce.FLCE_ERR_INVALID_ARG          # grad_bias without bias
    assert call(hidden=18) == flce.FLCE_ERR_UNSUPPORTED
    assert call(wsb=8) == flce.FLCE_ERR_WORKSPACE_TOO_SMALL


def test_scale_gradients_validation(lib):
    p = flce.make_params(64, 64, 100, reduction="sum")
    assert lib.flce_scale_gradients(ctypes.byref(p), None, 16, 16, None, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_scale_gradients(ctypes.byref(p), 16, 16, None, None, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_scale_gradients(ctypes.byref(p), 16, 18, 16, None, None) == flce.FLCE_ERR_UNSUPPORTED
    pn = flce.make_params(64, 64, 100, reduction="none")
    assert lib.flce_scale_gradients(ctypes.byref(pn), 16, 16, 16, None, None) == flce.FLCE_ERR_INVALID_ARG


def test_forward_no_alloc_refuses_problems_beyond_its_scratch(lib):
    """flce_forward_no_alloc keeps the forward scratch in a fixed 8 MiB array: a problem whose
    forward workspace is larger is refused on the host, before any HIP call."""
    big = flce.make_params(600_000, 64, 1000)
    assert _ws(big, flce.FLCE_PASS_FORWARD)[1] > 8 << 20
    assert lib.flce_forward_no_alloc(ctypes.byref(big), 16, 16, None, 16, 16, 16, None, None, None) == \
        flce.FLCE_ERR_UNSUPPORTED
    small = flce.make_params(64, 64, 100)
    assert lib.flce_forward_no_alloc(ctypes.byref(small), 16, None, None, 16, 16, 16, None, None, None) == \
        flce.FLCE_ERR_INVALID_ARG                     # NULL weight
    assert lib.flce_forward_no_alloc(ctypes.byref(small), 18, 16, None, 16, 16, 16, None, None, None) == \
        flce.FLCE_ERR_UNSUPPORTED                     # misaligned hidden
