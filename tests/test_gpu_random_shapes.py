"""GPU parity on a seeded sweep of small random shapes and options.

Each case draws N, H, V off the tile multiples (V down to 1, H down to 8), an
input dtype, bias or none, scale, softcap, z-loss, ignored rows, reduction and
the grad_weight dtype, and compares every output of flce_forward +
flce_backward with the fp64 oracle under the same tolerances as the fixed cases:
loss, LSE and entropy relative 2e-3 (16-bit) / 1e-5 (fp32), gradients
max |err| <= 1e-2 * max |ref|, num_correct exact outside near-tied rows.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_helpers import (LOSS_RTOL, assert_grad_close, assert_loss_close, assert_num_correct, t2np,
                         to_device, widened)

pytestmark = pytest.mark.gpu


@dataclasses.dataclass
class Shape:
    n: int
    h: int
    v: int
    dtype: str
    bias_std: float
    scale: float
    cap: float
    z_loss: float
    ignore_frac: float
    reduction: str
    gw_dtype: str
    weight_std: float
    seed: int
    vocab_chunk: int = 0

    @property
    def name(self):
        return (f"n{self.n}_h{self.h}_v{self.v}_{self.dtype}_{self.reduction}"
                f"{'_bias' if self.bias_std else ''}{'_cap' if self.cap else ''}"
                f"{f'_vc{self.vocab_chunk}' if self.vocab_chunk else ''}")


def _draw(count=16, seed=2026, n_min=1, n_max=900, h8_max=50, v_min=1, v_max=4000, chunks=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        n = int(np.exp(rng.uniform(np.log(n_min), np.log(n_max))))
        h = 8 * int(rng.integers(1, h8_max + 1))
        v = int(np.exp(rng.uniform(np.log(v_min), np.log(v_max))))
        dtype = ("bf16", "f16", "f32")[int(rng.integers(0, 3))]
        z_loss = 0.0 if rng.random() < 0.5 else 1e-3
        if v <= 1:
            # with one vocabulary row and no z-loss every gradient cancels to
            # exactly 0 (p = 1), which a rounded p need not reproduce bit for bit
            z_loss = 1e-3
        out.append(Shape(
            n=max(n, 1), h=h, v=max(v, 1), dtype=dtype,
            bias_std=0.1 if rng.random() < 0.5 else None,
            scale=1.0 if rng.random() < 0.5 else float(rng.uniform(0.3, 1.5)),
            cap=None if rng.random() < 0.5 else float(rng.uniform(1.5, 30.0)),
            z_loss=z_loss,
            ignore_frac=0.0 if rng.random() < 0.5 else 0.1,
            reduction=("sum", "mean", "none")[int(rng.integers(0, 3))],
            gw_dtype=None if rng.random() < 0.7 else "f32",
            weight_std=0.05 if rng.random() < 0.5 else 0.2,
            seed=seed % 1000 + i,
            # several vocabulary chunks in the backward pass (chunk width a
            # multiple of 256, at most the library's choice)
            vocab_chunk=256 * int(rng.integers(1, 9)) if chunks else 0))
    return out


# small shapes, down to N = 1, H = 8, V = 1; then mid sizes spanning several
# token tiles, vocabulary splits and backward chunks
SHAPES = _draw() + _draw(count=8, seed=77, n_min=300, n_max=3000, h8_max=100, v_min=1000, v_max=20000, chunks=True)


@pytest.mark.parametrize("c", SHAPES, ids=lambda c: c.name)
def test_random_shape_parity(flce_lib, c):
    import torch
    sys.stderr.write(f"[random] {c}\n")
    sys.stderr.flush()
    inp = si.make_inputs(c.n, c.h, c.v, dtype=c.dtype, weight_std=c.weight_std, bias_std=c.bias_std,
                         ignore_frac=c.ignore_frac, reduction=c.reduction, seed=c.seed)
    d = to_device(inp, c.dtype)
    opts = dict(logit_scale=c.scale, softcap=c.cap, z_loss=c.z_loss, reduction=c.reduction)
    loss, lse, met = flce_lib.forward(d["hidden"], d["weight"], d["targets"], d["bias"], return_metrics=True,
                                      **opts)
    g = d["grad_loss"] if c.reduction == "none" else d["grad_loss"][:1]
    gh, gw, gb = flce_lib.backward(d["hidden"], d["weight"], d["targets"], lse, g, d["bias"],
                                   grad_weight_dtype=c.gw_dtype, vocab_chunk=c.vocab_chunk, **opts)
    torch.cuda.synchronize()
    X, W, B, T = widened(inp, c.dtype)
    fwd, rgh, rgw, rgb = oracle.forward_backward(X, W, B, T, inp["grad_loss"].astype(np.float64), **opts)
    assert_loss_close(t2np(loss), fwd.loss, c.dtype, "loss")
    assert_loss_close(t2np(lse), fwd.lse, c.dtype, "lse")
    assert_num_correct(met["num_correct_tokens"].item(), fwd)
    ent = float(t2np(met["entropy_sum"]))
    if c.v == 1:
        # every entropy is 0: bound the cancellation in LSE - T/l by the LSE sizes
        assert abs(ent) <= LOSS_RTOL[c.dtype] * float(np.abs(fwd.lse[fwd.valid]).sum()) + 1e-30
    else:
        assert_loss_close(ent, fwd.entropy_sum, c.dtype, "entropy_sum")
    assert_grad_close(t2np(gh), rgh, "grad_hidden")
    assert_grad_close(t2np(gw), rgw, "grad_weight")
    if B is not None:
        assert_grad_close(t2np(gb), rgb, "grad_bias")
