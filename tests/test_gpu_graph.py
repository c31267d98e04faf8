"""flce_forward_no_alloc + flce_backward captured once in a HIP graph and
replayed: every replay, with eager work and synchronisations in between,
matches bitwise the eager calls on the same buffers -- also after the inputs'
contents change between replays (the graph re-reads them).  The two calls
enqueue kernels only (no memory set, copy or allocation), so they capture
as they are."""
import sys

import pytest

import synth_inputs as si
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def test_graph_capture_replays_match_eager(flce_lib):
    import torch
    flce = flce_lib
    n, h, v = 1000, 256, 5000
    opts = dict(logit_scale=0.8, softcap=20.0, z_loss=1e-4, reduction="mean")
    sys.stderr.write(f"[graph] N={n} H={h} V={v}\n")
    sys.stderr.flush()
    inputs = []
    for seed in (41, 42):
        inp = si.make_inputs(n, h, v, dtype="bf16", weight_std=0.1, bias_std=0.1, ignore_frac=0.1,
                             reduction="mean", seed=seed)
        inputs.append(to_device(inp, "bf16"))
    # the buffers the graph is bound to, filled from input set 0
    d = {k: (t.clone() if t is not None else None) for k, t in inputs[0].items()}
    p = flce.make_params(n, h, v, dtype="bf16", **opts)
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    loss = torch.empty(1, device="cuda")
    lse = torch.empty(n, device="cuda")
    nc = torch.empty(1, dtype=torch.int64, device="cuda")
    ent = torch.empty(1, device="cuda")
    gh = torch.empty(n, h, dtype=torch.bfloat16, device="cuda")
    gw = torch.empty(v, h, dtype=torch.bfloat16, device="cuda")
    gb = torch.empty(v, dtype=torch.bfloat16, device="cuda")
    gl = d["grad_loss"][:1].clone()
    ws = torch.empty(flce.flce_workspace_size(p, flce.FLCE_PASS_BACKWARD), dtype=torch.uint8, device="cuda")
    outs = (loss, lse, nc, ent, gh, gw, gb)

    def step():
        st = torch.cuda.current_stream().cuda_stream
        rc = flce.flce_forward_no_alloc(p, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]),
                                        P(loss), P(lse), P(nc), P(ent), st)
        assert rc == 0, flce.status_string(rc)
        rc = flce.flce_backward(p, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]), P(lse), P(gl),
                                P(gh), P(gw), P(gb), P(ws), ws.numel(), st)
        assert rc == 0, flce.status_string(rc)

    def load(k):
        for key in ("hidden", "weight", "bias", "targets"):
            d[key].copy_(inputs[k][key])
        torch.cuda.synchronize()

    refs = []
    for k in (0, 1):
        load(k)
        step()
        torch.cuda.synchronize()
        refs.append([o.clone() for o in outs])
    assert not torch.equal(refs[0][4], refs[1][4])

    load(0)
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                   # warm-up on the capture stream's kind of stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    names = ("loss", "lse", "num_correct", "entropy_sum", "grad_hidden", "grad_weight", "grad_bias")
    for rep, k in enumerate((0, 0, 1, 0, 1, 1)):
        load(k)
        for o in outs:                     # eager work between replays: sentinels in every output
            o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, r in zip(names, outs, refs[k]):
            assert torch.equal(o, r), f"replay {rep} (inputs {k}): {name}"
