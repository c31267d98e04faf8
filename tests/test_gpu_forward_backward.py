"""GPU parity of the one-pass forward + backward (flce_forward_backward: the
row-chunked schedule, gradients formed from each block's stored logits)
against the fp64 oracle, with the tolerances of the two-call path: loss, LSE
and entropy relative 2e-3 (bf16) / 1e-5 (fp32); gradients max |err| <=
1e-2 * max |ref|; num_correct exact except for near-tied rows.  Blocks of 256
rows force several blocks (and a ragged last one) at these sizes."""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_helpers import assert_grad_close, assert_loss_close, assert_num_correct, t2np, to_device, widened
from test_gpu_parity import RAGGED_MID, SMALL_CASES, Case, _inputs, _opts, _sampled_check, _say

pytestmark = pytest.mark.gpu


def _run_fused(flce, c: Case, d: dict, block_rows=0, **kw):
    import torch
    g = d["grad_loss"] if c.reduction == "none" else d["grad_loss"][:1]
    out = flce.forward_backward(d["hidden"], d["weight"], d["targets"], g, d["bias"], grad_weight_dtype=c.gw_dtype,
                                return_metrics=True, block_rows=block_rows, **_opts(c), **kw)
    torch.cuda.synchronize()
    return out


def _check_against_oracle(c, inp, out, grad_tol_note=""):
    loss, lse, met, gh, gw, gb = out
    X, W, B, T = widened(inp, c.dtype)
    fwd, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **_opts(c))
    assert_loss_close(t2np(loss), fwd.loss, c.dtype, "loss")
    assert_loss_close(t2np(lse), fwd.lse, c.dtype, "lse")
    assert_num_correct(met["num_correct_tokens"].item(), fwd)
    assert_loss_close(t2np(met["entropy_sum"]), fwd.entropy_sum, c.dtype, "entropy_sum")
    assert_grad_close(t2np(gh), rgh, "grad_hidden" + grad_tol_note)
    assert_grad_close(t2np(gw), rgw, "grad_weight" + grad_tol_note)
    if B is not None:
        assert_grad_close(t2np(gb), rgb, "grad_bias" + grad_tol_note)
    return rgh, rgw, rgb


# The one-pass path forms its gradients from logits stored in the input dtype
# (16-bit for 16-bit inputs), so p = exp(z - LSE) carries that rounding: fine
# for logits of a few tens (a softcap of 30 or less), off by tens of percent for
# logits in the hundreds (bf16 rounds z = 500 to a multiple of 2).  Those cases
# check its fp32 outputs only (below); the two-call path covers them in full.
HUGE_LOGITS = [c for c in SMALL_CASES if c.name.startswith("huge_logits")]
ONE_PASS_CASES = [c for c in SMALL_CASES if c not in HUGE_LOGITS]


@pytest.mark.parametrize("block_rows", [0, 256])
@pytest.mark.parametrize("case", ONE_PASS_CASES, ids=lambda c: c.name)
def test_forward_backward_parity(flce_lib, case, block_rows):
    c = case
    _say(f"[fused] {c.name} N={c.n} H={c.h} V={c.v} {c.dtype} {c.reduction} block_rows={block_rows}")
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    _check_against_oracle(c, inp, _run_fused(flce_lib, c, d, block_rows))


@pytest.mark.parametrize("case", HUGE_LOGITS, ids=lambda c: c.name)
def test_forward_backward_huge_logits_fp32_outputs(flce_lib, case):
    """Logits in the hundreds: loss, LSE and the metrics come from the fp32 tile state
    and stay within tolerance; the gradients are out of this path's range (above)."""
    c = case
    _say(f"[one-pass] {c.name} N={c.n} H={c.h} V={c.v} (fp32 outputs only)")
    inp = _inputs(c)
    loss, lse, met, gh, gw, gb = _run_fused(flce_lib, c, to_device(inp, c.dtype))
    X, W, B, T = widened(inp, c.dtype)
    fwd = oracle.forward(X, W, B, T, **_opts(c))
    assert_loss_close(t2np(loss), fwd.loss, c.dtype, "loss")
    assert_loss_close(t2np(lse), fwd.lse, c.dtype, "lse")
    assert_num_correct(met["num_correct_tokens"].item(), fwd)
    assert_loss_close(t2np(met["entropy_sum"]), fwd.entropy_sum, c.dtype, "entropy_sum")


@pytest.mark.parametrize("h", [72, 256])
def test_forward_backward_accumulates(flce_lib, h):
    """FLCE_ACCUMULATE_GRAD_WEIGHT / _BIAS over several blocks (bf16 grad_weight: the fp32
    accumulator's last block adds the prior contents); H = 256 takes the epilogue form for
    blocks inside the matrix."""
    import torch
    c = Case("fused_accumulate", 700, h, 3000, "bf16", 0.1, 0.8, 3.0, 1e-3, 0.1, "mean", weight_std=0.1, seed=23)
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    X, W, B, T = widened(inp, c.dtype)
    _, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **_opts(c))
    rng = np.random.default_rng(6)
    gw0 = si.widen(si.round_to_bf16_bits(rng.normal(0, np.abs(rgw).max() / 4, (c.v, c.h)).astype(np.float32)), "bf16")
    gb0 = si.widen(si.round_to_bf16_bits(rng.normal(0, np.abs(rgb).max() / 4, c.v).astype(np.float32)), "bf16")
    gw_buf = torch.from_numpy(gw0.astype(np.float32)).to(torch.bfloat16).cuda()
    gb_buf = torch.from_numpy(gb0.astype(np.float32)).to(torch.bfloat16).cuda()
    loss, lse, met, gh, gw, gb = _run_fused(flce_lib, c, d, 256, grad_weight=gw_buf, grad_bias=gb_buf)
    assert gw.data_ptr() == gw_buf.data_ptr() and gb.data_ptr() == gb_buf.data_ptr()
    assert_grad_close(t2np(gh), rgh, "grad_hidden")
    assert_grad_close(t2np(gw) - gw0, rgw, "grad_weight (accumulated, minus prior)")
    assert_grad_close(t2np(gb) - gb0, rgb, "grad_bias (accumulated, minus prior)")


def test_forward_backward_matches_two_calls(flce_lib):
    """Loss, LSE and metrics come from the same fp32 tile state as flce_forward: they agree
    with the two-call path to rounding; the gradients to the parity tolerance."""
    import torch
    from test_gpu_parity import _run_gpu
    c = Case("fused_vs_split", 1000, 256, 5000, "bf16", 0.1, 0.5, 30.0, 0.0, 0.05, "sum", weight_std=0.05, seed=3)
    d = to_device(_inputs(c), c.dtype)
    a = _run_gpu(flce_lib, c, d)
    b = _run_fused(flce_lib, c, d, 256)
    assert abs(a[0].item() - b[0].item()) <= 1e-5 * abs(a[0].item())
    assert torch.allclose(a[1], b[1], rtol=1e-6, atol=1e-6)
    assert a[2]["num_correct_tokens"].item() == b[2]["num_correct_tokens"].item()
    for name, x, y in (("grad_hidden", a[3], b[3]), ("grad_weight", a[4], b[4]), ("grad_bias", a[5], b[5])):
        x, y = x.float(), y.float()
        assert (x - y).abs().max().item() <= 1e-2 * x.abs().max().item(), name


@pytest.mark.parametrize("reduction", ["sum", "mean", "none"])
def test_forward_backward_empty_batch(flce_lib, reduction):
    import torch
    dev = "cuda"
    h, v = 64, 300
    hidden = torch.empty((0, h), dtype=torch.bfloat16, device=dev)
    weight = torch.randn((v, h), device=dev).to(torch.bfloat16)
    bias = torch.randn(v, device=dev).to(torch.bfloat16)
    targets = torch.empty(0, dtype=torch.int64, device=dev)
    g = torch.ones(1, dtype=torch.float32, device=dev)
    loss, lse, met, gh, gw, gb = flce_lib.forward_backward(hidden, weight, targets, g, bias, reduction=reduction,
                                                          return_metrics=True)
    torch.cuda.synchronize()
    if reduction == "sum":
        assert loss.item() == 0.0
    elif reduction == "mean":
        assert torch.isnan(loss).item()
    assert met["num_correct_tokens"].item() == 0
    assert gh.numel() == 0 and not gw.any().item() and not gb.any().item()


def test_forward_backward_all_rows_ignored_mean(flce_lib):
    import torch
    c = Case("fused_all_ignored", 600, 64, 500, "bf16", 0.1, reduction="mean", weight_std=0.1)
    inp = _inputs(c)
    inp["targets"][:] = si.IGNORE_INDEX
    d = to_device(inp, c.dtype)
    loss, lse, met, gh, gw, gb = _run_fused(flce_lib, c, d, 256)
    assert torch.isnan(loss).item()
    assert met["num_correct_tokens"].item() == 0 and met["entropy_sum"].item() == 0.0
    assert not gh.any().item() and not gw.any().item() and not gb.any().item()


def test_forward_backward_f16_small_gradients(flce_lib):
    """fp16 with "mean" over ~1350 valid rows, V = 40000, in six blocks: each block picks its
    own power-of-two factor for the stored logit gradient (and grad_bias sums the unscaled
    values), so the error stays at the scaled level (~3e-4), far below the ~1.2e-2 of an
    unscaled fp16 gradient."""
    c = Case("f16_mean_small_gradients", 1500, 128, 40000, "f16", 0.1, 1.0, None, 1e-3, 0.1, "mean", weight_std=0.05)
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    loss, lse, met, gh, gw, gb = _run_fused(flce_lib, c, d, 256)
    X, W, B, T = widened(inp, c.dtype)
    _, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **_opts(c))
    for what, a, r in (("grad_hidden", t2np(gh), rgh), ("grad_weight", t2np(gw), rgw), ("grad_bias", t2np(gb), rgb)):
        err = np.abs(a - r).max() / np.abs(r).max()
        assert err <= 2e-3, f"{what}: {err:.3e}"


@pytest.mark.slow
@pytest.mark.parametrize("name", ["bf16_n8192_h4096_v128256", "bf16_n16384_h2048_v256000",
                                  "bf16_n8192_h4096_v32000_zipf", "f16_n8192_h4096_v128256"])
def test_forward_backward_full_size_sampled(flce_lib, name):
    _sampled_check(flce_lib, si.WORKLOADS[name], run=lambda f, c, d: _run_fused(f, c, d, 0))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_forward_backward_int32_targets(flce_lib, dtype):
    """int32 targets give the same bits as the same targets in int64 (several blocks)."""
    import torch
    c = Case("fused_int32_targets", 700, 200, 1500, dtype, 0.1, 0.7, 2.0, 0.01, 0.1, "mean", weight_std=0.1)
    d = to_device(_inputs(c), c.dtype)
    r64 = _run_fused(flce_lib, c, d, 256)
    d32 = dict(d)
    d32["targets"] = d["targets"].to(torch.int32)
    r32 = _run_fused(flce_lib, c, d32, 256)
    for name, a, b in zip(("loss", "lse", "grad_hidden", "grad_weight", "grad_bias"),
                          (r64[0], r64[1], r64[3], r64[4], r64[5]), (r32[0], r32[1], r32[3], r32[4], r32[5])):
        assert torch.equal(a, b), name
    assert r64[2]["num_correct_tokens"].item() == r32[2]["num_correct_tokens"].item()


def test_forward_backward_deterministic(flce_lib):
    """Same inputs, same bits, run to run (no float atomics anywhere)."""
    import torch
    c = Case("fused_determinism", 600, 192, 3000, "bf16", 0.1, 0.8, 8.0, 1e-3, 0.1, "sum", weight_std=0.1)
    d = to_device(_inputs(c), c.dtype)
    a = _run_fused(flce_lib, c, d, 256)
    b = _run_fused(flce_lib, c, d, 256)
    for i, name in ((0, "loss"), (1, "lse"), (3, "grad_hidden"), (4, "grad_weight"), (5, "grad_bias")):
        assert torch.equal(a[i], b[i]), name
    assert torch.equal(a[2]["entropy_sum"], b[2]["entropy_sum"])


def test_forward_backward_grad_weight_accumulated_in_weight_dtype(flce_lib):
    """grad_weight_accum_dtype="weight" (FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT): the blocks' grad_weight
    contributions are summed in bf16, rounding after each of the three blocks; still within the
    gradient tolerance, and not bitwise the fp32-accumulated result."""
    import torch
    c = Case("fused_accum_weight_dtype", 700, 256, 3000, "bf16", 0.1, 0.8, 3.0, 1e-3, 0.1, "mean", weight_std=0.1,
             seed=29)
    inp = _inputs(c)
    d = to_device(inp, c.dtype)
    out_w = _run_fused(flce_lib, c, d, 256, grad_weight_accum_dtype="weight")
    rgh, rgw, rgb = _check_against_oracle(c, inp, out_w)
    out_f = _run_fused(flce_lib, c, d, 256)
    assert torch.equal(out_w[3], out_f[3])            # grad_hidden does not depend on it
    assert not torch.equal(out_w[4], out_f[4])


@pytest.mark.slow
def test_forward_backward_ragged_mid_size_sampled(flce_lib):
    """N=6000, H=1600, V=50257, every option on, in blocks of 2048 rows: three blocks, the last
    ragged, the fp32 grad_weight partial carried across them."""
    _sampled_check(flce_lib, RAGGED_MID, run=lambda f, c, d: _run_fused(f, c, d, 2048))
