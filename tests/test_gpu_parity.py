"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Small and medium cases compare every output element; the full-size workloads
compare sampled gradient rows with the oracle's LSE computed for every row.
Tolerances: loss, LSE and entropy relative 2e-3 (bf16) / 1e-5 (fp32);
gradients max |err| <= 1e-2 * max |ref|; num_correct exact except for rows
whose two largest oracle logits are closer than 1e-3.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_helpers import (LOSS_RTOL, assert_grad_close, assert_loss_close, assert_num_correct, t2np,
                         to_device, widened)

LOSS_RTOL_BF16 = LOSS_RTOL["bf16"]

pytestmark = pytest.mark.gpu


def _say(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


@dataclasses.dataclass
class Case:
    name: str
    n: int
    h: int
    v: int
    dtype: str = "bf16"
    bias_std: float = None
    scale: float = 1.0
    cap: float = None
    z_loss: float = 0.0
    ignore_frac: float = 0.0
    reduction: str = "mean"
    gw_dtype: str = None
    targets: str = "uniform"
    weight_std: float = 0.02
    seed: int = 11


def _from_workload(wl: si.Workload) -> Case:
    return Case(wl.name, wl.n_tokens, wl.hidden, wl.vocab, wl.dtype, wl.bias_std, wl.logit_scale,
                wl.softcap, wl.z_loss, wl.ignore_frac, wl.reduction, wl.grad_weight_dtype, wl.targets,
                wl.weight_std, wl.seed)


SMALL_CASES = [
    _from_workload(si.WORKLOADS["tiny_fp32"]),
    _from_workload(si.WORKLOADS["bf16_n2048_h1024_v32000"]),
    # several tiles in every dimension, ragged tails (N, V not multiples of 256,
    # H not a multiple of the 64-wide K stage), every option on
    Case("ragged_bf16_all_options", 700, 200, 1500, "bf16", 0.1, 0.7, 2.0, 0.01, 0.1, "mean",
         weight_std=0.1),
    Case("ragged_bf16_none_gwf32", 333, 136, 777, "bf16", None, 1.0, None, 0.0, 0.05, "none", "f32",
         weight_std=0.1),
    Case("ragged_f32_sum_softcap", 300, 72, 1000, "f32", 0.2, 0.5, 5.0, 0.001, 0.0, "sum",
         weight_std=0.1),
    Case("vocab_smaller_than_tile", 513, 64, 37, "bf16", 0.1, 1.0, None, 0.0, 0.0, "sum",
         weight_std=0.2),
    Case("single_row", 1, 128, 300, "bf16", 0.1, 1.3, 10.0, 0.0, 0.0, "mean", weight_std=0.1),
    # more than one vocabulary chunk in the backward pass (chunk <= 32768 rows)
    Case("two_vocab_chunks_bias", 256, 64, 40000, "bf16", 0.1, 1.0, None, 1e-3, 0.1, "mean",
         weight_std=0.1),
    Case("zipf_targets_zloss", 1024, 256, 5000, "bf16", None, 1.0, None, 1e-4, 0.0, "mean",
         targets="zipf", weight_std=0.05),
    # fp16 inputs: the same ragged shapes and options, fp16 or fp32 grad_weight
    Case("ragged_f16_all_options", 700, 200, 1500, "f16", 0.1, 0.7, 2.0, 0.01, 0.1, "mean",
         weight_std=0.1),
    Case("ragged_f16_none_gwf32", 333, 136, 777, "f16", None, 1.0, None, 0.0, 0.05, "none", "f32",
         weight_std=0.1),
    # logits in the hundreds without a cap: every exponential is taken relative
    # to the running maximum (p is nearly one-hot, LSE ~ the row maximum)
    Case("huge_logits_no_cap", 300, 64, 1000, "bf16", 0.1, 200.0, None, 0.0, 0.05, "sum", weight_std=0.1),
    Case("huge_logits_no_cap_f16_zloss", 300, 64, 1000, "f16", 0.1, 200.0, None, 1e-4, 0.05, "mean",
         weight_std=0.1),
    # H = 8: one K stage, all but its first 16 (bf16) or 32 (fp32) bytes per row
    # past the end of the rows
    Case("hidden_8_bf16", 600, 8, 3000, "bf16", 0.1, 1.0, None, 0.0, 0.05, "sum", weight_std=0.3),
    Case("hidden_8_f32", 300, 8, 700, "f32", None, 1.0, 3.0, 1e-3, 0.0, "none", weight_std=0.3),
    # fp16 with "mean" over ~1350 valid rows and V = 40000 (two vocabulary
    # chunks): the off-target logit gradients are ~2e-8, below fp16's smallest
    # subnormal, unless the backward scales them (a dropped scale fails here)
    Case("f16_mean_small_gradients", 1500, 128, 40000, "f16", 0.1, 1.0, None, 1e-3, 0.1, "mean",
         weight_std=0.05),
]


def _inputs(c: Case):
    return si.make_inputs(c.n, c.h, c.v, dtype=c.dtype, weight_std=c.weight_std, bias_std=c.bias_std,
                          targets=c.targets, ignore_frac=c.ignore_frac, reduction=c.reduction,
                          seed=c.seed)


def _opts(c: Case):
    return dict(logit_scale=c.scale, softcap=c.cap, z_loss=c.z_loss, reduction=c.reduction)


def _run_gpu(flce, c: Case, d: dict, return_metrics=True):
    import torch
    loss, lse, met = flce.forward(d["hidden"], d["weight"], d["targets"], d["bias"],
                                  return_metrics=return_metrics, **_opts(c))
    g = d["grad_loss"] if c.reduction == "none" else d["grad_loss"][:1]
    gh, gw, gb = flce.backward(d["hidden"], d["weight"], d["targets"], lse, g, d["bias"],
                               grad_weight_dtype=c.gw_dtype, **_opts(c))
    torch.cuda.synchronize()
    return loss, lse, met, gh, gw, gb


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: c.name)
def test_full_parity(flce_lib, case):
    c = case
    _say(f"[parity] {c.name} N={c.n} H={c.h} V={c.v} {c.dtype} {c.reduction}")
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    loss, lse, met, gh, gw, gb = _run_gpu(flce_lib, c, d)
    X, W, B, T = widened(inp, c.dtype)
    fwd, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64),
                                                 **_opts(c))
    assert_loss_close(t2np(loss), fwd.loss, c.dtype, "loss")
    assert_loss_close(t2np(lse), fwd.lse, c.dtype, "lse")
    assert_num_correct(met["num_correct_tokens"].item(), fwd)
    assert_loss_close(t2np(met["entropy_sum"]), fwd.entropy_sum, c.dtype, "entropy_sum")
    assert_grad_close(t2np(gh), rgh, "grad_hidden")
    assert_grad_close(t2np(gw), rgw, "grad_weight")
    if B is not None:
        assert_grad_close(t2np(gb), rgb, "grad_bias")
    assert flce_lib.get_status(_ws_probe(flce_lib, d)) == 0


def test_vocabulary_of_one(flce_lib):
    """V = 1 (255 of the tile's 256 vocabulary rows past the end): LSE = z, the loss is
    the z-loss alone, every valid row counts as correct, the entropy is 0 up to the
    cancellation in LSE - T/l, and the gradients are 2 lam c z times the chain."""
    c = Case("vocab_one", 300, 64, 1, "bf16", 0.1, 0.8, 4.0, 1e-2, 0.1, "mean", weight_std=0.1)
    _say(f"[parity] {c.name} N={c.n} H={c.h} V={c.v}")
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    loss, lse, met, gh, gw, gb = _run_gpu(flce_lib, c, d)
    X, W, B, T = widened(inp, c.dtype)
    fwd, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64),
                                                 **_opts(c))
    assert fwd.num_correct == fwd.n_valid
    assert_loss_close(t2np(loss), fwd.loss, c.dtype, "loss")
    assert_loss_close(t2np(lse), fwd.lse, c.dtype, "lse")
    assert met["num_correct_tokens"].item() == fwd.n_valid
    # entropy_i = LSE_i - T_i / l_i: each term is of size |LSE_i|, the difference 0
    ent = float(t2np(met["entropy_sum"]))
    bound = LOSS_RTOL_BF16 * float(np.abs(fwd.lse[fwd.valid]).sum())
    assert abs(ent) <= bound, f"entropy_sum {ent:.3e} beyond {bound:.3e}"
    assert_grad_close(t2np(gh), rgh, "grad_hidden")
    assert_grad_close(t2np(gw), rgw, "grad_weight")
    assert_grad_close(t2np(gb), rgb, "grad_bias")


def _ws_probe(flce, d):
    """A freshly written forward workspace whose status word reflects `d`'s targets."""
    import torch
    n, h = d["hidden"].shape
    dt = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[d["hidden"].dtype]
    p = flce.make_params(n, h, d["weight"].shape[0], dtype=dt, reduction="sum")
    ws = torch.empty(flce.flce_workspace_size(p, flce.FLCE_PASS_FORWARD), dtype=torch.uint8,
                     device=d["hidden"].device)
    loss, lse, _ = flce.forward(d["hidden"], d["weight"], d["targets"], d["bias"], reduction="sum",
                                workspace=ws)
    return ws


@pytest.mark.parametrize("h", [72, 256])
@pytest.mark.parametrize("gw_dtype", ["bf16", "f32"])
def test_accumulate_into_grad_weight_and_bias(flce_lib, gw_dtype, h):
    """FLCE_ACCUMULATE_GRAD_WEIGHT / _BIAS: the backward adds to the buffers' contents
    (two vocabulary chunks, so every chunk's grad_weight rows take the add).  H = 72 leaves
    every wave's block partly outside the matrix, H = 256 puts most inside (the two
    epilogue forms)."""
    import torch
    c = Case("accumulate", 300, h, 33000, "bf16", 0.1, 0.8, 3.0, 1e-3, 0.1, "mean", gw_dtype,
             weight_std=0.1, seed=21)
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    loss, lse, _ = flce_lib.forward(d["hidden"], d["weight"], d["targets"], d["bias"], **_opts(c))
    X, W, B, T = widened(inp, c.dtype)
    _, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **_opts(c))
    # seeded prior contents on the gradients' scale (so that rounding the sum once stays
    # inside the gradient tolerance), exactly representable in the buffers' dtypes
    rng = np.random.default_rng(5)
    sw, sb = np.abs(rgw).max() / 4, np.abs(rgb).max() / 4
    gw0 = si.widen(si.round_to_bf16_bits(rng.normal(0, sw, (c.v, c.h)).astype(np.float32)), "bf16")
    gb0 = si.widen(si.round_to_bf16_bits(rng.normal(0, sb, c.v).astype(np.float32)), "bf16")
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    gw_buf = torch.from_numpy(gw0.astype(np.float32)).to(tdt[gw_dtype]).cuda()
    gb_buf = torch.from_numpy(gb0.astype(np.float32)).to(torch.bfloat16).cuda()
    g = d["grad_loss"][:1]
    gh, gw, gb = flce_lib.backward(d["hidden"], d["weight"], d["targets"], lse, g, d["bias"],
                                   grad_weight=gw_buf, grad_bias=gb_buf, **_opts(c))
    torch.cuda.synchronize()
    assert gw.data_ptr() == gw_buf.data_ptr() and gb.data_ptr() == gb_buf.data_ptr()
    assert_grad_close(t2np(gh), rgh, "grad_hidden")
    assert_grad_close(t2np(gw) - gw0, rgw, "grad_weight (accumulated, minus prior)")
    assert_grad_close(t2np(gb) - gb0, rgb, "grad_bias (accumulated, minus prior)")


def test_all_rows_ignored_mean(flce_lib):
    import torch
    c = Case("all_ignored", 300, 64, 500, "bf16", 0.1, reduction="mean", weight_std=0.1)
    inp = _inputs(c)
    inp["targets"][:] = si.IGNORE_INDEX
    d = to_device(inp, c.dtype)
    loss, lse, met, gh, gw, gb = _run_gpu(flce_lib, c, d)
    assert torch.isnan(loss).item()
    assert met["num_correct_tokens"].item() == 0 and met["entropy_sum"].item() == 0.0
    assert not gh.any().item() and not gw.any().item() and not gb.any().item()
    X, W, B, T = widened(inp, c.dtype)
    fwd = oracle.forward(X, W, B, T, reduction="mean")
    assert_loss_close(t2np(lse), fwd.lse, "bf16", "lse")


@pytest.mark.parametrize("reduction", ["sum", "mean", "none"])
def test_empty_batch(flce_lib, reduction):
    import torch
    dev = "cuda"
    h, v = 64, 300
    hidden = torch.empty((0, h), dtype=torch.bfloat16, device=dev)
    weight = torch.randn((v, h), device=dev).to(torch.bfloat16)
    bias = torch.randn(v, device=dev).to(torch.bfloat16)
    targets = torch.empty(0, dtype=torch.int64, device=dev)
    loss, lse, met = flce_lib.forward(hidden, weight, targets, bias, reduction=reduction,
                                      return_metrics=True)
    g = torch.ones(1 if reduction != "none" else 0, dtype=torch.float32, device=dev)
    if reduction == "none":
        g = torch.ones(1, dtype=torch.float32, device=dev)
    gh, gw, gb = flce_lib.backward(hidden, weight, targets, lse, g, bias, reduction=reduction)
    torch.cuda.synchronize()
    if reduction == "sum":
        assert loss.item() == 0.0
    elif reduction == "mean":
        assert torch.isnan(loss).item()
    assert met["num_correct_tokens"].item() == 0
    assert gh.numel() == 0 and not gw.any().item() and not gb.any().item()


def test_deterministic_and_metrics_bit_identical(flce_lib):
    import torch
    c = Case("determinism", 600, 192, 3000, "bf16", 0.1, 0.8, 8.0, 1e-3, 0.1, "sum", weight_std=0.1)
    d = to_device(_inputs(c), c.dtype)
    a = _run_gpu(flce_lib, c, d, return_metrics=True)
    b = _run_gpu(flce_lib, c, d, return_metrics=False)
    for x, y, name in ((a[0], b[0], "loss"), (a[1], b[1], "lse"), (a[3], b[3], "grad_hidden"),
                       (a[4], b[4], "grad_weight"), (a[5], b[5], "grad_bias")):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x, y.view(torch.uint8)
                           if y.dtype == torch.bfloat16 else y), f"{name} differs between runs"
    a2 = _run_gpu(flce_lib, c, d, return_metrics=True)
    assert torch.equal(a[2]["num_correct_tokens"], a2[2]["num_correct_tokens"])
    assert torch.equal(a[2]["entropy_sum"], a2[2]["entropy_sum"])


def test_argmax_ties_take_lowest_index(flce_lib):
    import torch
    n, h, v = 256, 64, 600
    rng = np.random.default_rng(5)
    x = np.ones((n, h), dtype=np.float32)
    w = (rng.standard_normal((v, h)) * 0.01).astype(np.float32)
    w[5] = 0.1
    w[9] = 0.1          # rows 5 and 9 tie for the maximum on every token
    w[300] = 0.1        # and so does a row in another 256-wide tile
    t = np.where(np.arange(n) % 3 == 0, 5, np.where(np.arange(n) % 3 == 1, 9, 300)).astype(np.int64)
    inp = {"hidden": si.round_to_bf16_bits(x), "weight": si.round_to_bf16_bits(w), "bias": None,
           "targets": t, "grad_loss": np.array(1.0, dtype=np.float32)}
    d = to_device(inp, "bf16")
    _, _, met = flce_lib.forward(d["hidden"], d["weight"], d["targets"], None, reduction="sum",
                                 return_metrics=True)
    assert met["num_correct_tokens"].item() == int((t == 5).sum())


def test_out_of_range_target_sets_status(flce_lib):
    import torch
    c = Case("oob", 300, 64, 500, "bf16", None, reduction="sum", weight_std=0.1)
    inp = _inputs(c)
    inp["targets"][7] = 500          # == V: out of range
    d = to_device(inp, c.dtype)
    p = flce_lib.make_params(c.n, c.h, c.v, reduction="sum")
    ws = torch.empty(flce_lib.flce_workspace_size(p, flce_lib.FLCE_PASS_FORWARD), dtype=torch.uint8,
                     device="cuda")
    loss, lse, _ = flce_lib.forward(d["hidden"], d["weight"], d["targets"], None, reduction="sum",
                                    workspace=ws)
    assert flce_lib.get_status(ws) == flce_lib.FLCE_ERR_TARGET_OUT_OF_RANGE
    # the row is treated as ignored
    t = inp["targets"].copy()
    t[7] = si.IGNORE_INDEX
    X, W, B, _ = widened(inp, c.dtype)
    fwd = oracle.forward(X, W, B, t, reduction="sum")
    assert_loss_close(t2np(loss), fwd.loss, "bf16")
    wsb = torch.empty(flce_lib.flce_workspace_size(p, flce_lib.FLCE_PASS_BACKWARD), dtype=torch.uint8,
                      device="cuda")
    gh, gw, _ = flce_lib.backward(d["hidden"], d["weight"], d["targets"], lse,
                                  torch.ones(1, device="cuda"), None, reduction="sum", workspace=wsb)
    assert flce_lib.get_status(wsb) == flce_lib.FLCE_ERR_TARGET_OUT_OF_RANGE
    assert not gh[7].any().item()


def test_host_validation_errors(flce_lib):
    import torch
    x = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(16, dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        flce_lib.forward(x, w, t, reduction="bogus")
    p_bad = flce_lib.make_params(16, 64, 100)
    p_bad.reduction = 7
    out = torch.empty(16, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    assert flce_lib.flce_forward(p_bad, x.data_ptr(), w.data_ptr(), None, t.data_ptr(), out.data_ptr(),
                                 out.data_ptr(), None, None, ws.data_ptr(), ws.numel(),
                                 None) == flce_lib.FLCE_ERR_INVALID_ARG
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = flce_lib.make_params(16, 64, 100)
    out = torch.empty(1, device="cuda")
    rc = flce_lib.flce_forward(p, x.data_ptr(), w.data_ptr(), None, t.data_ptr(), out.data_ptr(),
                               out.data_ptr(), None, None, small_ws.data_ptr(), 16, None)
    assert rc == flce_lib.FLCE_ERR_WORKSPACE_TOO_SMALL


# ----------------------------------------------------------------------------- large workloads

def _sampled_check(flce, wl: si.Workload, n_rows=512, n_vocab=512, run=None):
    import torch
    c = _from_workload(wl)
    _say(f"[parity-large] {wl.name}: drawing inputs")
    inp = si.make_workload_inputs(wl)
    d = to_device(inp, c.dtype)
    _say(f"[parity-large] {wl.name}: GPU forward+backward")
    loss, lse, met, gh, gw, gb = (run or _run_gpu)(flce, c, d)
    loss_n, lse_n = t2np(loss), t2np(lse)
    nc, ent = met["num_correct_tokens"].item(), met["entropy_sum"].item()
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(c.n, n_rows, replace=False))
    ign = np.nonzero(inp["targets"] == si.IGNORE_INDEX)[0]
    if ign.size:
        rows[:4] = ign[:4]
        rows = np.unique(rows)
    valid_t = inp["targets"][inp["targets"] != si.IGNORE_INDEX]
    vids = np.unique(np.concatenate([rng.choice(c.v, min(n_vocab // 2, c.v), replace=False),
                                     rng.choice(valid_t, n_vocab // 2)]))
    gh_s = t2np(gh[torch.from_numpy(rows).cuda()])
    gw_s = t2np(gw[torch.from_numpy(vids).cuda()])
    gb_n = t2np(gb)
    del gh, gw, d
    torch.cuda.empty_cache()
    grad_loss = inp["grad_loss"].astype(np.float64)
    X, W, B, T = widened(inp, c.dtype)
    del inp["weight"]
    _say(f"[parity-large] {wl.name}: oracle pass over all rows")
    fwd, rgb = oracle.full_pass_with_bias_grad(X, W, B, T, grad_loss, **_opts(c))
    assert_loss_close(loss_n, fwd.loss, c.dtype, "loss")
    assert_loss_close(lse_n, fwd.lse, c.dtype, "lse")
    assert_num_correct(nc, fwd)
    assert_loss_close(ent, fwd.entropy_sum, c.dtype, "entropy_sum")
    if B is not None:
        assert_grad_close(gb_n, rgb, "grad_bias")
    _say(f"[parity-large] {wl.name}: oracle sampled gradients")
    rgh, rgw = oracle.sampled_gradients(X, W, B, T, grad_loss, fwd.lse, rows, vids, **_opts(c))
    assert_grad_close(gh_s, rgh, "grad_hidden (sampled rows)")
    assert_grad_close(gw_s, rgw, "grad_weight (sampled vocab rows)")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["bf16_n8192_h4096_v128256", "bf16_n16384_h2048_v256000",
                                  "bf16_n8192_h4096_v32000_zipf", "f16_n8192_h4096_v128256"])
def test_full_size_sampled(flce_lib, name):
    _sampled_check(flce_lib, si.WORKLOADS[name])


# Everything ragged at a mid size: N, H and V none a multiple of 256 (H = 1600
# leaves a partial hidden tile in both gradient contractions), an odd V (the
# bias staging rounds its last word), all options on, and the cap low enough
# to bend the logits.
RAGGED_MID = si.Workload("bf16_n6000_h1600_v50257_ragged", 6000, 1600, 50257, "bf16", 0.02, 0.1,
                         logit_scale=0.8, softcap=5.0, z_loss=1e-4, ignore_frac=0.1, reduction="mean",
                         seed=7)


@pytest.mark.slow
def test_ragged_mid_size_sampled(flce_lib):
    _sampled_check(flce_lib, RAGGED_MID)


# The largest hidden the boundary accepts: N*H*2 bytes = 2^31 - 64 KiB (every
# 32-bit byte range the kernels form, and the 2 GiB transposed copy of hidden,
# at their limit); a small vocabulary keeps the oracle's full pass to seconds.
MAX_ROWS = si.Workload("bf16_n262136_h4096_v64_max_rows", 262136, 4096, 64, "bf16", 0.05, 0.1,
                       logit_scale=0.5, softcap=30.0, ignore_frac=0.05, reduction="sum", seed=9)


@pytest.mark.slow
def test_max_rows_sampled(flce_lib):
    _sampled_check(flce_lib, MAX_ROWS)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_int32_targets_match_int64(flce_lib, dtype):
    """int32 targets (FLCE_TARGETS_INT32) give bit-identical results to the same targets as int64."""
    import torch
    c = Case("int32_targets", 700, 200, 1500, dtype, 0.1, 0.7, 2.0, 0.01, 0.1, "mean", weight_std=0.1)
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    r64 = _run_gpu(flce_lib, c, d)
    d32 = dict(d)
    d32["targets"] = d["targets"].to(torch.int32)
    r32 = _run_gpu(flce_lib, c, d32)
    for name, a, b in zip(("loss", "lse", "grad_hidden", "grad_weight", "grad_bias"),
                          (r64[0], r64[1], r64[3], r64[4], r64[5]), (r32[0], r32[1], r32[3], r32[4], r32[5])):
        assert torch.equal(a, b), name
    assert r64[2]["num_correct_tokens"].item() == r32[2]["num_correct_tokens"].item()
    assert torch.equal(r64[2]["entropy_sum"], r32[2]["entropy_sum"])
    X, W, B, T = widened(inp, c.dtype)
    fwd = oracle.forward(X, W, B, T, **_opts(c))
    assert_loss_close(t2np(r32[0]), fwd.loss, c.dtype, "loss")


def test_f16_small_gradients_keep_precision(flce_lib):
    """fp16 logit gradients under "mean" with V = 40000: the entries are ~2e-8, below fp16's
    subnormals; rounded unscaled they put grad_bias and grad_hidden off by ~1.2e-2 of their
    maximum (an fp64 emulation of that rounding), scaled by a power of two by ~3e-4.  Bound
    2e-3 separates the two with a wide margin."""
    c = Case("f16_mean_small_gradients", 1500, 128, 40000, "f16", 0.1, 1.0, None, 1e-3, 0.1, "mean",
             weight_std=0.05)
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    loss, lse, met, gh, gw, gb = _run_gpu(flce_lib, c, d)
    X, W, B, T = widened(inp, c.dtype)
    _, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **_opts(c))
    for what, a, r in (("grad_hidden", t2np(gh), rgh), ("grad_weight", t2np(gw), rgw), ("grad_bias", t2np(gb), rgb)):
        err = np.abs(a - r).max() / np.abs(r).max()
        assert err <= 2e-3, f"{what}: {err:.3e}"


def test_autograd_function(flce_lib):
    """linear_cross_entropy under torch autograd: the loss and the leaf gradients equal the
    direct flce_forward / flce_backward calls with the upstream gradient autograd passes
    (here 2.5 for "sum", a vector for "none")."""
    import torch
    for red in ("sum", "none"):
        c = Case("autograd", 300, 136, 1100, "bf16", 0.1, 0.8, 4.0, 1e-3, 0.1, red, weight_std=0.1, seed=17)
        d = to_device(_inputs(c), c.dtype)
        x = d["hidden"].clone().requires_grad_(True)
        w = d["weight"].clone().requires_grad_(True)
        b = d["bias"].clone().requires_grad_(True)
        loss = flce_lib.linear_cross_entropy(x, w, d["targets"], b, **_opts(c))
        up = torch.full((), 2.5, device="cuda") if red == "sum" else torch.linspace(-1, 1, c.n, device="cuda")
        (loss * up).sum().backward()
        l2, lse, _ = flce_lib.forward(d["hidden"], d["weight"], d["targets"], d["bias"], **_opts(c))
        g = up.reshape(1) if red == "sum" else up
        gh, gw, gb = flce_lib.backward(d["hidden"], d["weight"], d["targets"], lse, g.float().contiguous(),
                                       d["bias"], **_opts(c))
        torch.cuda.synchronize()
        assert torch.equal(loss.detach(), l2)
        assert torch.equal(x.grad, gh) and torch.equal(w.grad, gw) and torch.equal(b.grad, gb)


def test_autograd_one_pass(flce_lib):
    """linear_cross_entropy(one_pass=True): gradients precomputed with an upstream gradient of 1,
    scaled in backward by the one autograd passes (2.5 here, and 1); they match the two-call op's
    within the gradient tolerance; "none" is refused, and so is a second backward."""
    import torch
    for red, up in (("sum", 2.5), ("mean", 1.0)):
        c = Case("autograd_one_pass", 700, 136, 1100, "bf16", 0.1, 0.8, 4.0, 1e-3, 0.1, red, weight_std=0.1, seed=19)
        d = to_device(_inputs(c), c.dtype)
        grads = []
        for one_pass in (False, True):
            x = d["hidden"].clone().requires_grad_(True)
            w = d["weight"].clone().requires_grad_(True)
            b = d["bias"].clone().requires_grad_(True)
            loss = flce_lib.linear_cross_entropy(x, w, d["targets"], b, one_pass=one_pass, **_opts(c))
            (loss * up).backward()
            torch.cuda.synchronize()
            grads.append((loss.detach(), x.grad, w.grad, b.grad))
        (l0, *g0), (l1, *g1) = grads
        assert abs(l0.item() - l1.item()) <= 1e-5 * abs(l0.item())
        for name, a, r in zip(("grad_hidden", "grad_weight", "grad_bias"), g1, g0):
            assert_grad_close(t2np(a), t2np(r), name)
    c = Case("autograd_one_pass_none", 300, 64, 500, "bf16", reduction="none", weight_std=0.1)
    d = to_device(_inputs(c), c.dtype)
    with pytest.raises(ValueError):
        flce_lib.linear_cross_entropy(d["hidden"], d["weight"], d["targets"], reduction="none", one_pass=True)
    x = d["hidden"].clone().requires_grad_(True)
    loss = flce_lib.linear_cross_entropy(x, d["weight"], d["targets"], reduction="sum", one_pass=True)
    loss.backward(retain_graph=True)
    with pytest.raises(RuntimeError):
        loss.backward()
