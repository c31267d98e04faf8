"""The Python binding checks dtypes, shapes and devices before anything is
launched (CPU only: every case raises before the library is called).  The
kernels read weight and bias in hidden's dtype with hidden's row length and
trust the lengths of targets, lse and the upstream gradient, so each mismatch
below would otherwise read or write out of bounds, or misread silently."""
import pytest
import torch

import linear_cross_entropy_tiled_amd as flce

N, H, V = 16, 64, 100


def _args(dtype=torch.bfloat16):
    return dict(hidden=torch.zeros(N, H, dtype=dtype), weight=torch.zeros(V, H, dtype=dtype),
                targets=torch.zeros(N, dtype=torch.int64), bias=torch.zeros(V, dtype=dtype))


@pytest.mark.parametrize("change,exc", [
    (dict(weight=torch.zeros(V, H, dtype=torch.float32)), TypeError),       # fp32 weight, bf16 hidden
    (dict(bias=torch.zeros(V, dtype=torch.float32)), TypeError),            # fp32 bias under AMP
    (dict(weight=torch.zeros(V, H + 8, dtype=torch.bfloat16)), ValueError),  # wrong width
    (dict(bias=torch.zeros(V - 1, dtype=torch.bfloat16)), ValueError),
    (dict(targets=torch.zeros(N - 1, dtype=torch.int64)), ValueError),       # short targets
    (dict(targets=torch.zeros(N, dtype=torch.float32)), TypeError),
    (dict(hidden=torch.zeros(N, H, dtype=torch.float64)), TypeError),
    (dict(hidden=torch.zeros(N, H, 2, dtype=torch.bfloat16)), ValueError),
    (dict(hidden=torch.zeros(H, N, dtype=torch.bfloat16).t()), ValueError),  # not contiguous
    (dict(), ValueError),                                                    # consistent, but on the CPU
])
def test_forward_rejects(change, exc):
    a = _args()
    a.update(change)
    with pytest.raises(exc):
        flce.forward(a["hidden"], a["weight"], a["targets"], a["bias"], reduction="sum")


@pytest.mark.parametrize("change,exc", [
    (dict(lse=torch.zeros(N - 1)), ValueError),
    (dict(lse=torch.zeros(N, dtype=torch.float64)), TypeError),
    (dict(grad_loss=torch.ones(2)), ValueError),                    # "sum" takes one value
    (dict(grad_loss=torch.ones(1, dtype=torch.bfloat16)), TypeError),
    (dict(grad_weight=torch.zeros(V, H - 8)), ValueError),
    (dict(grad_bias=torch.zeros(V, dtype=torch.float32)), TypeError),
    (dict(grad_bias=torch.zeros(V + 1, dtype=torch.bfloat16)), ValueError),
    (dict(), ValueError),
])
def test_backward_rejects(change, exc):
    a = _args()
    b = dict(lse=torch.zeros(N), grad_loss=torch.ones(1), grad_weight=None, grad_bias=None)
    b.update(change)
    with pytest.raises(exc):
        flce.backward(a["hidden"], a["weight"], a["targets"], b["lse"], b["grad_loss"], a["bias"],
                      reduction="sum", grad_weight=b["grad_weight"], grad_bias=b["grad_bias"])


def test_none_reduction_needs_one_upstream_value_per_row():
    a = _args()
    with pytest.raises(ValueError):
        flce.backward(a["hidden"], a["weight"], a["targets"], torch.zeros(N), torch.ones(1), a["bias"],
                      reduction="none")
    with pytest.raises(ValueError):
        flce.forward_backward(a["hidden"], a["weight"], a["targets"], torch.ones(1), a["bias"], reduction="none")


def test_grad_bias_without_bias_and_bad_reduction():
    a = _args()
    with pytest.raises(ValueError):
        flce.backward(a["hidden"], a["weight"], a["targets"], torch.zeros(N), torch.ones(1), None,
                      reduction="sum", grad_bias=torch.zeros(V, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        flce.forward(a["hidden"], a["weight"], a["targets"], a["bias"], reduction="avg")


def test_chunked_path_rejects_mismatches():
    x = torch.zeros(N, H, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        flce.weighted_mse(x, torch.zeros(V, H, dtype=torch.float16), torch.zeros(N, V), torch.ones(N),
                          torch.ones(V))
    with pytest.raises(ValueError):
        flce.chunked_linear_loss(x, torch.zeros(V, H + 8, dtype=torch.bfloat16), lambda z: (z.sum(), z))
