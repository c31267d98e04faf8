"""flce_forward_no_alloc (the forward pass with its scratch in a fixed device
array inside the library, for callers that cannot allocate) against
flce_forward with a workspace: the same kernels, so the same bits, on two calls
in a row -- the second with a smaller problem, which reuses the array the first
one left behind."""
import sys

import numpy as np
import pytest

import synth_inputs as si
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _run_both(flce, n, h, v, seed, **opts):
    import torch
    sys.stderr.write(f"[no_alloc] N={n} H={h} V={v}\n")
    sys.stderr.flush()
    inp = si.make_inputs(n, h, v, dtype="bf16", weight_std=0.1, bias_std=0.1, ignore_frac=0.1,
                         reduction=opts["reduction"], seed=seed, plant_frac=0.5, plant_margin=12.0)
    d = to_device(inp, "bf16")
    p = flce.make_params(n, h, v, dtype="bf16", **opts)
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for no_alloc in (False, True):
        loss = torch.full((n if opts["reduction"] == "none" else 1,), -1.0, device="cuda")
        lse = torch.full((n,), -1.0, device="cuda")
        nc = torch.full((1,), -1, dtype=torch.int64, device="cuda")
        ent = torch.full((1,), -1.0, device="cuda")
        if no_alloc:
            rc = flce.flce_forward_no_alloc(p, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]),
                                            P(loss), P(lse), P(nc), P(ent), stream)
        else:
            ws = torch.empty(flce.flce_workspace_size(p, flce.FLCE_PASS_FORWARD), dtype=torch.uint8, device="cuda")
            rc = flce.flce_forward(p, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]), P(loss),
                                   P(lse), P(nc), P(ent), P(ws), ws.numel(), stream)
        assert rc == 0, flce.status_string(rc)
        torch.cuda.synchronize()
        outs.append((loss, lse, nc, ent))
    for name, a, b in zip(("loss", "lse", "num_correct", "entropy_sum"), outs[0], outs[1]):
        assert torch.equal(a, b), name
    assert outs[1][2].item() > 0.3 * n * 0.9     # planted rows: the count is far from 0


def test_no_alloc_forward_matches_forward_on_two_calls(flce_lib):
    opts = dict(logit_scale=0.8, softcap=6.0, z_loss=1e-3, reduction="mean")
    # the first call: 12 token tiles x 21 splits of partials; the second, smaller (3 tiles, 85 splits)
    _run_both(flce_lib, 3000, 256, 20000, 71, **opts)
    _run_both(flce_lib, 700, 200, 50000, 72, **opts)


def test_no_alloc_forward_none_reduction(flce_lib):
    _run_both(flce_lib, 513, 136, 3000, 73, logit_scale=1.0, softcap=None, z_loss=0.0, reduction="none")
