"""Two problems in flight at once on two streams (each call with its own
workspace, outputs and the stream current at the call) give bitwise the results
of the same calls made one after the other: the library keeps no state between
calls, and the kernels of one call touch only that call's buffers."""
import numpy as np
import pytest

import synth_inputs as si
from gpu_helpers import t2np, to_device

pytestmark = pytest.mark.gpu


def _problem(seed, n, h, v):
    inp = si.make_inputs(n, h, v, dtype="bf16", weight_std=0.1, bias_std=0.1, ignore_frac=0.05,
                         reduction="sum", seed=seed)
    return to_device(inp, "bf16")


def _step(flce, d):
    opts = dict(logit_scale=0.7, softcap=20.0, z_loss=1e-4, reduction="sum")
    loss, lse, met = flce.forward(d["hidden"], d["weight"], d["targets"], d["bias"], return_metrics=True, **opts)
    gh, gw, gb = flce.backward(d["hidden"], d["weight"], d["targets"], lse, d["grad_loss"][:1], d["bias"],
                               **opts)
    return [loss, lse, met["num_correct_tokens"], met["entropy_sum"], gh, gw, gb]


def test_two_streams_match_sequential(flce_lib):
    import torch
    a = _problem(31, 1500, 384, 9000)
    b = _problem(32, 700, 256, 40000)   # two vocabulary chunks
    ref_a = [t2np(t) for t in _step(flce_lib, a)]
    ref_b = [t2np(t) for t in _step(flce_lib, b)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    torch.cuda.current_stream().synchronize()
    for rep in range(3):
        with torch.cuda.stream(s1):
            out_a = _step(flce_lib, a)
        with torch.cuda.stream(s2):
            out_b = _step(flce_lib, b)
        torch.cuda.synchronize()
        for name, x, r in zip(("loss", "lse", "num_correct", "entropy_sum", "grad_hidden", "grad_weight",
                               "grad_bias"), out_a, ref_a):
            assert np.array_equal(t2np(x), r, equal_nan=True), f"stream 1, {name}, repetition {rep}"
        for name, x, r in zip(("loss", "lse", "num_correct", "entropy_sum", "grad_hidden", "grad_weight",
                               "grad_bias"), out_b, ref_b):
            assert np.array_equal(t2np(x), r, equal_nan=True), f"stream 2, {name}, repetition {rep}"
