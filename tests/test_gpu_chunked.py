"""GPU parity of the generic chunked linear loss (flce_chunked_linear_loss)
against the fp64 oracle, through the C ABI: the built-in weighted squared
error (the "Chunked Linear Loss" page's direct-gradient example), a loss
function written in Python, error propagation and grad_weight accumulation."""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_helpers import assert_grad_close, assert_loss_close, t2np

pytestmark = pytest.mark.gpu


def _say(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


@dataclasses.dataclass
class WCase:
    name: str
    n: int
    h: int
    v: int
    dtype: str = "bf16"
    chunk_rows: int = 0
    gw_dtype: str = None
    accum: str = "fp32"
    weight_std: float = 0.1
    seed: int = 3


CASES = [
    # several row blocks with a ragged last one, ragged V and H
    WCase("ragged_bf16_blocks", 700, 200, 1500, "bf16", chunk_rows=256),
    WCase("ragged_f16_blocks", 700, 200, 1500, "f16", chunk_rows=256),
    WCase("f32_blocks", 300, 72, 1000, "f32", chunk_rows=256),
    WCase("one_block_small_vocab", 513, 64, 37, "bf16"),
    WCase("bf16_gw_f32", 600, 128, 3000, "bf16", chunk_rows=256, gw_dtype="f32"),
    # grad_weight summed in bf16 across the blocks ("weight" accumulation)
    WCase("bf16_accum_weight", 600, 128, 3000, "bf16", chunk_rows=256, accum="weight"),
    WCase("mid_bf16_4_blocks", 2048, 1024, 32000, "bf16", chunk_rows=512, weight_std=0.02),
]


def _dev(inp, dtype):
    import torch
    def d(a):
        if dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return {k: d(v) for k, v in inp.items()}


def _case_inputs(c):
    return si.make_wmse_inputs(c.n, c.h, c.v, dtype=c.dtype, weight_std=c.weight_std, seed=c.seed)


def _oracle(inp, dtype):
    x = si.widen(inp["hidden"], dtype)
    w = si.widen(inp["weight"], dtype)
    return oracle.weighted_mse(x, w, inp["target"].astype(np.float64), inp["row_weight"].astype(np.float64),
                               inp["feature_weight"].astype(np.float64))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_weighted_mse_parity(flce_lib, case):
    import torch
    c = case
    _say(f"[chunked] {c.name} N={c.n} H={c.h} V={c.v} {c.dtype} rows/block={c.chunk_rows}")
    inp = _case_inputs(c)
    d = _dev(inp, c.dtype)
    loss, gi, gw = flce_lib.weighted_mse(d["hidden"], d["weight"], d["target"], d["row_weight"],
                                         d["feature_weight"], chunk_rows=c.chunk_rows,
                                         grad_weight_dtype=c.gw_dtype, grad_weight_accum_dtype=c.accum)
    torch.cuda.synchronize()
    r_loss, r_gi, r_gw = _oracle(inp, c.dtype)
    assert_loss_close(t2np(loss), r_loss, c.dtype, "loss")
    assert_grad_close(t2np(gi), r_gi, "grad_inputs")
    assert_grad_close(t2np(gw), r_gw, "grad_weight")


def test_python_loss_function_matches_builtin(flce_lib):
    """The same weighted squared error written with torch ops in a Python loss
    function gives the built-in kernel's results."""
    import torch
    c = WCase("python_fn", 700, 200, 1500, "bf16", chunk_rows=256)
    inp = _case_inputs(c)
    d = _dev(inp, c.dtype)

    def wmse(logits, target, row_weight, feature_weight):
        err = logits.float() - target
        w = row_weight[:, None] * feature_weight[None, :]
        return (err * err * w).sum(), (2 * err * w).to(logits.dtype)

    loss_p, gi_p, gw_p = flce_lib.chunked_linear_loss(d["hidden"], d["weight"], wmse, d["target"], d["row_weight"],
                                                      d["feature_weight"], chunk_rows=256)
    loss_b, gi_b, gw_b = flce_lib.weighted_mse(d["hidden"], d["weight"], d["target"], d["row_weight"],
                                               d["feature_weight"], chunk_rows=256)
    torch.cuda.synchronize()
    assert abs(loss_p.item() - loss_b.item()) <= 1e-5 * abs(loss_b.item())
    assert_grad_close(t2np(gi_p), t2np(gi_b), "grad_inputs (python vs built-in)")
    assert_grad_close(t2np(gw_p), t2np(gw_b), "grad_weight (python vs built-in)")
    r_loss, r_gi, r_gw = _oracle(inp, c.dtype)
    assert_loss_close(t2np(loss_p), r_loss, c.dtype, "loss")
    assert_grad_close(t2np(gi_p), r_gi, "grad_inputs")


def test_loss_function_error_is_reported(flce_lib):
    import torch
    x = torch.zeros((300, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((500, 64), dtype=torch.bfloat16, device="cuda")

    class Boom(Exception):
        pass

    calls = []

    def bad(logits):
        calls.append(logits.shape)
        raise Boom("loss function failed")

    with pytest.raises(Boom):
        flce_lib.chunked_linear_loss(x, w, bad, chunk_rows=256)
    torch.cuda.synchronize()
    assert calls == [(256, 500)]   # stopped after the first block


def test_accumulate_into_grad_weight(flce_lib):
    import torch
    c = WCase("accumulate", 600, 128, 3000, "bf16", chunk_rows=256)
    inp = _case_inputs(c)
    d = _dev(inp, c.dtype)
    r_loss, r_gi, r_gw = _oracle(inp, c.dtype)
    rng = np.random.default_rng(9)
    prior = rng.normal(0, np.abs(r_gw).max() / 4, r_gw.shape).astype(np.float32)
    buf = torch.from_numpy(prior).cuda()
    loss, gi, gw = flce_lib.weighted_mse(d["hidden"], d["weight"], d["target"], d["row_weight"],
                                         d["feature_weight"], chunk_rows=256, grad_weight=buf)
    torch.cuda.synchronize()
    assert gw.data_ptr() == buf.data_ptr()
    assert_grad_close(t2np(gw) - prior, r_gw, "grad_weight (accumulated, minus prior)")


def test_empty_inputs(flce_lib):
    import torch
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((100, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((0, 100), dtype=torch.float32, device="cuda")
    r = torch.zeros(0, dtype=torch.float32, device="cuda")
    f = torch.ones(100, dtype=torch.float32, device="cuda")
    loss, gi, gw = flce_lib.weighted_mse(x, w, y, r, f)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and gi.numel() == 0
    assert not gw.any().item()
