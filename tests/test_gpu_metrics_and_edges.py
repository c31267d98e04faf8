"""GPU parity for the argmax metric at sizes where it can fail, and edge cases of
the backward's padding and of the "mean" reduction.

* num_correct (fused-linear-ce README, "Metrics for free"): inputs with planted
  targets (about half of the rows' hidden vectors carry a component along their
  target's weight row), so that the oracle's count is a large share of the valid
  rows and the allowance for near-ties is tiny; the maxima then sit in every
  vocabulary split, and a kernel that returned 0 or merged the splits wrongly
  fails.  A constructed case puts exact ties across vocabulary splits far from
  the first one.
* Padding rows (N not a multiple of 256) with logits large enough that an
  unguarded exp overflows: every gradient stays finite and matches the oracle.
* "mean" over valid rows ("Chunked Linear Loss", "Reduction semantics") with the
  ignored rows clustered in one 256-row tile, or spread one per row block.
"""
import sys

import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_helpers import (assert_grad_close, assert_loss_close, assert_num_correct, t2np, to_device,
                         widened)

pytestmark = pytest.mark.gpu


def _say(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def _opts(scale=1.0, cap=None, z_loss=0.0, reduction="mean"):
    return dict(logit_scale=scale, softcap=cap, z_loss=z_loss, reduction=reduction)


def _full_check(flce, inp, dtype, opts, min_frac=None):
    import torch
    d = to_device(inp, dtype)
    loss, lse, met = flce.forward(d["hidden"], d["weight"], d["targets"], d["bias"], return_metrics=True, **opts)
    g = d["grad_loss"] if opts["reduction"] == "none" else d["grad_loss"][:1]
    gh, gw, gb = flce.backward(d["hidden"], d["weight"], d["targets"], lse, g, d["bias"], **opts)
    torch.cuda.synchronize()
    X, W, B, T = widened(inp, dtype)
    fwd, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **opts)
    assert_num_correct(met["num_correct_tokens"].item(), fwd, min_frac=min_frac)
    assert_loss_close(t2np(loss), fwd.loss, dtype, "loss")
    assert_loss_close(t2np(lse), fwd.lse, dtype, "lse")
    assert_loss_close(t2np(met["entropy_sum"]), fwd.entropy_sum, dtype, "entropy_sum")
    for name, a, r in (("grad_hidden", gh, rgh), ("grad_weight", gw, rgw), ("grad_bias", gb, rgb)):
        if r is not None:
            a = t2np(a)
            assert np.isfinite(a).all(), f"{name} has non-finite entries"
            assert_grad_close(a, r, name)
    return fwd


def test_num_correct_planted_n2048_h1024_v32000(flce_lib):
    """The 2048-token, 32000-vocabulary recipe (10% ignored, mean) with half the rows planted."""
    _say("[metrics] planted N=2048 H=1024 V=32000")
    inp = si.make_inputs(2048, 1024, 32000, dtype="bf16", weight_std=0.02, ignore_frac=0.1, reduction="mean",
                         seed=1, plant_frac=0.5)
    fwd = _full_check(flce_lib, inp, "bf16", _opts(), min_frac=0.3)
    _say(f"[metrics] oracle num_correct {fwd.num_correct} of {fwd.n_valid}")


def test_num_correct_planted_ragged_many_splits(flce_lib):
    """Three token tiles (the last ragged) over 196 vocabulary tiles: the forward pass splits the
    vocabulary 85 ways, so most maxima lie far from the first split; bias, scale and cap on."""
    _say("[metrics] planted N=700 H=200 V=50000, 85 splits")
    inp = si.make_inputs(700, 200, 50000, dtype="bf16", weight_std=0.1, bias_std=0.1, ignore_frac=0.1,
                         reduction="sum", seed=12, plant_frac=0.5, plant_margin=12.0)
    _full_check(flce_lib, inp, "bf16", _opts(scale=0.7, cap=6.0, z_loss=1e-3, reduction="sum"), min_frac=0.3)


@pytest.mark.slow
def test_num_correct_planted_headline_shape(flce_lib):
    """The headline recipe (N=8192, H=4096, V=128256, bias, scale 0.5, cap 30, 5% ignored, sum)
    with half the rows planted: loss, LSE, metrics and grad_bias over every row, gradients on
    sampled rows, as the full-size parity test does."""
    import torch
    wl = si.WORKLOADS["bf16_n8192_h4096_v128256"]
    _say("[metrics] planted headline shape: drawing inputs")
    inp = si.make_inputs(wl.n_tokens, wl.hidden, wl.vocab, dtype=wl.dtype, weight_std=wl.weight_std,
                         bias_std=wl.bias_std, ignore_frac=wl.ignore_frac, reduction=wl.reduction, seed=wl.seed,
                         plant_frac=0.5)
    opts = _opts(wl.logit_scale, wl.softcap, wl.z_loss, wl.reduction)
    d = to_device(inp, wl.dtype)
    _say("[metrics] planted headline shape: GPU forward + backward")
    loss, lse, met = flce_lib.forward(d["hidden"], d["weight"], d["targets"], d["bias"], return_metrics=True, **opts)
    gh, gw, gb = flce_lib.backward(d["hidden"], d["weight"], d["targets"], lse, d["grad_loss"][:1], d["bias"], **opts)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = np.sort(rng.choice(wl.n_tokens, 256, replace=False))
    vids = np.unique(np.concatenate([rng.choice(wl.vocab, 128, replace=False),
                                     rng.choice(inp["targets"][inp["targets"] >= 0], 128)]))
    res = dict(loss=t2np(loss), lse=t2np(lse), nc=met["num_correct_tokens"].item(),
               ent=met["entropy_sum"].item(), gb=t2np(gb), gh=t2np(gh[torch.from_numpy(rows).cuda()]),
               gw=t2np(gw[torch.from_numpy(vids).cuda()]))
    del d, gh, gw
    torch.cuda.empty_cache()
    X, W, B, T = widened(inp, wl.dtype)
    _say("[metrics] planted headline shape: oracle pass over all rows")
    g = inp["grad_loss"].astype(np.float64)
    fwd, rgb = oracle.full_pass_with_bias_grad(X, W, B, T, g, **opts)
    _say(f"[metrics] oracle num_correct {fwd.num_correct} of {fwd.n_valid}, GPU {res['nc']}")
    assert_num_correct(res["nc"], fwd, min_frac=0.3)
    assert_loss_close(res["loss"], fwd.loss, wl.dtype, "loss")
    assert_loss_close(res["lse"], fwd.lse, wl.dtype, "lse")
    assert_loss_close(res["ent"], fwd.entropy_sum, wl.dtype, "entropy_sum")
    assert_grad_close(res["gb"], rgb, "grad_bias")
    rgh, rgw = oracle.sampled_gradients(X, W, B, T, g, fwd.lse, rows, vids, **opts)
    assert_grad_close(res["gh"], rgh, "grad_hidden (sampled rows)")
    assert_grad_close(res["gw"], rgw, "grad_weight (sampled vocab rows)")


def test_argmax_exact_ties_across_late_splits(flce_lib):
    """One-hot hidden rows (token i has a 1 at feature i % 64) and a weight whose column k is
    small noise except two exactly equal maxima, at vocabulary rows a_k < b_k in different,
    late vocabulary splits (the forward pass splits 20000 rows into 128 parts here).  The
    lowest-index rule makes a_k the argmax: tokens whose target is a_k count, those whose
    target is b_k do not."""
    import torch
    n, h, v = 512, 64, 20000
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((v, h)) * 0.01).astype(np.float32)
    a = 10000 + 37 * np.arange(h)          # split ~64 onwards
    b = a + 5000 + 11 * np.arange(h)       # a later split still
    w[a, np.arange(h)] = 0.5
    w[b, np.arange(h)] = 0.5
    x = np.zeros((n, h), dtype=np.float32)
    x[np.arange(n), np.arange(n) % h] = 1.0
    k = np.arange(n) % h
    t = np.where(np.arange(n) % 3 == 2, b[k], a[k]).astype(np.int64)
    inp = {"hidden": si.round_to_bf16_bits(x), "weight": si.round_to_bf16_bits(w), "bias": None, "targets": t,
           "grad_loss": np.array(1.0, dtype=np.float32)}
    d = to_device(inp, "bf16")
    _, _, met = flce_lib.forward(d["hidden"], d["weight"], d["targets"], None, reduction="sum", return_metrics=True)
    torch.cuda.synchronize()
    X, W, B, T = widened(inp, "bf16")
    fwd = oracle.forward(X, W, B, T, reduction="sum")
    assert (fwd.argmax == a[k]).all() and fwd.num_correct == int((np.arange(n) % 3 != 2).sum())
    assert met["num_correct_tokens"].item() == fwd.num_correct


@pytest.mark.parametrize("cap", [None, 20.0])
def test_padding_rows_with_large_logits_stay_finite(flce_lib, cap):
    """N = 700 (the last token tile has 68 padding rows), scale 1, and a bias of ~100 on a few
    vocabulary rows: the padding rows' logits are the bias alone, and an exp against a zero
    LSE would overflow there.  Loss and all gradients are finite and match the oracle."""
    inp = si.make_inputs(700, 128, 3000, dtype="bf16", weight_std=0.05, bias_std=0.1, ignore_frac=0.1,
                         reduction="mean", seed=31)
    bias = si.widen(inp["bias"], "bf16")
    bias[[3, 700, 2999]] = [100.0, 96.0, 104.0]
    inp["bias"] = si.round_to_bf16_bits(bias.astype(np.float32))
    _full_check(flce_lib, inp, "bf16", _opts(cap=cap))


@pytest.mark.parametrize("layout", ["one_tile", "spread"])
def test_mean_with_clustered_ignored_rows(flce_lib, layout):
    """"mean" is the global sum over valid rows divided by their number, whatever the tiles and
    row blocks: ignored rows all in the second 256-row tile, or spread one per 256-row block.
    Both entry points (two calls; one pass with several block sizes) match the oracle, and the
    one-pass gradients agree with the two-call ones."""
    import torch
    n, h, v = 1100, 136, 4000
    inp = si.make_inputs(n, h, v, dtype="bf16", weight_std=0.1, bias_std=0.1, reduction="mean", seed=41)
    t = inp["targets"]
    if layout == "one_tile":
        t[256:512] = si.IGNORE_INDEX
    else:
        t[np.arange(0, n, 256) + 17] = si.IGNORE_INDEX
    opts = _opts(scale=0.9, cap=8.0, z_loss=1e-3)
    fwd = _full_check(flce_lib, inp, "bf16", opts)
    X, W, B, T = widened(inp, "bf16")
    assert float(fwd.loss) == pytest.approx(float(fwd.row_loss.sum()) / fwd.n_valid, rel=1e-15)
    d = to_device(inp, "bf16")
    one = torch.ones(1, device="cuda")
    _, lse, _ = flce_lib.forward(d["hidden"], d["weight"], d["targets"], d["bias"], **opts)
    gh0, gw0, gb0 = flce_lib.backward(d["hidden"], d["weight"], d["targets"], lse, one, d["bias"], **opts)
    for br in (256, 512, 0):
        loss, _, _, gh, gw, gb = flce_lib.forward_backward(d["hidden"], d["weight"], d["targets"], one, d["bias"],
                                                           block_rows=br, **opts)
        torch.cuda.synchronize()
        assert_loss_close(t2np(loss), fwd.loss, "bf16", f"one-pass mean, block_rows={br}")
        for name, a, r in (("grad_hidden", gh, gh0), ("grad_weight", gw, gw0), ("grad_bias", gb, gb0)):
            assert_grad_close(t2np(a), t2np(r), f"{name} one pass (block_rows={br}) vs two calls")


def test_timed_entry_points_record_every_launch_and_change_nothing(flce_lib):
    """flce_forward_timed / flce_backward_timed: bit-identical outputs to the untimed calls, one
    event pair per matrix-core launch (the forward tile kernel, then dlogits, grad_weight and
    grad_hidden per vocabulary chunk: 5 chunks of at most 1024 rows here), positive durations."""
    import torch
    n, h, v = 700, 200, 5000
    inp = si.make_inputs(n, h, v, dtype="bf16", weight_std=0.1, bias_std=0.1, ignore_frac=0.1, reduction="sum",
                         seed=51)
    d = to_device(inp, "bf16")
    opts = _opts(scale=0.8, cap=5.0, z_loss=1e-3, reduction="sum")
    p = flce_lib.make_params(n, h, v, dtype="bf16", vocab_chunk=1024, **opts)
    stream = torch.cuda.current_stream()
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    outs = []
    for timed in (False, True):
        ws_f = torch.empty(flce_lib.flce_workspace_size(p, flce_lib.FLCE_PASS_FORWARD), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(flce_lib.flce_workspace_size(p, flce_lib.FLCE_PASS_BACKWARD), dtype=torch.uint8, device="cuda")
        loss = torch.empty(1, device="cuda")
        lse = torch.empty(n, device="cuda")
        gh = torch.empty((n, h), dtype=torch.bfloat16, device="cuda")
        gw = torch.empty((v, h), dtype=torch.bfloat16, device="cuda")
        gb = torch.empty(v, dtype=torch.bfloat16, device="cuda")
        timer = flce_lib.LaunchTimer(capacity=32, stream=stream) if timed else None
        tc = timer.c if timed else None
        assert flce_lib.flce_forward_timed(p, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]), P(loss),
                                           P(lse), None, None, P(ws_f), ws_f.numel(), stream.cuda_stream, tc) == 0
        assert flce_lib.flce_backward_timed(p, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]), P(lse),
                                            P(d["grad_loss"][:1]), P(gh), P(gw), P(gb), P(ws_b), ws_b.numel(),
                                            stream.cuda_stream, tc) == 0
        torch.cuda.synchronize()
        outs.append((loss, lse, gh, gw, gb))
        if timed:
            assert timer.c.count == 1 + 3 * 5
            kinds = [timer._kinds[k] for k in range(timer.c.count)]
            assert kinds == [flce_lib.FLCE_KERNEL_FORWARD_TILES] + [flce_lib.FLCE_KERNEL_DLOGITS,
                                                                    flce_lib.FLCE_KERNEL_GRAD_WEIGHT,
                                                                    flce_lib.FLCE_KERNEL_GRAD_HIDDEN] * 5
            dur = timer.durations()
            assert sorted(dur) == sorted(flce_lib.KERNEL_NAMES.values())
            assert all(x > 0 for ms in dur.values() for x in ms)
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("vocab_chunk", [256, 1280, 0])
def test_vocab_chunk_parity(flce_lib, vocab_chunk):
    """The backward with chunks of 256 (21 chunks), 1280 (the last one short) and the library's
    width (one chunk) against the oracle."""
    import torch
    n, h, v = 600, 136, 5300
    inp = si.make_inputs(n, h, v, dtype="bf16", weight_std=0.1, bias_std=0.1, ignore_frac=0.1, reduction="mean",
                         seed=61)
    opts = _opts(scale=0.8, cap=5.0, z_loss=1e-3)
    d = to_device(inp, "bf16")
    _, lse, _ = flce_lib.forward(d["hidden"], d["weight"], d["targets"], d["bias"], **opts)
    gh, gw, gb = flce_lib.backward(d["hidden"], d["weight"], d["targets"], lse, d["grad_loss"][:1], d["bias"],
                                   vocab_chunk=vocab_chunk, **opts)
    torch.cuda.synchronize()
    X, W, B, T = widened(inp, "bf16")
    _, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **opts)
    assert_grad_close(t2np(gh), rgh, "grad_hidden")
    assert_grad_close(t2np(gw), rgw, "grad_weight")
    assert_grad_close(t2np(gb), rgb, "grad_bias")
