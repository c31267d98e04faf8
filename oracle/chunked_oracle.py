"""fp64 CPU oracle for the generic chunked linear loss.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's
``cpu_baseline`` leg may import this module; it shares no code with the HIP
path.

The generic path of the "Chunked Linear Loss" page computes, block of rows by
block of rows, logits = inputs @ weight.T, hands each block to a function that
returns the block's loss and the gradient of the loss with respect to the
logits, and then forms grad_input[block] = grad_logits @ weight and
grad_weight += grad_logits.T @ inputs[block] ("Why chunk the projection?",
"Loss function contract").  Losses that add up over rows give the same result
with one block holding every row, which is what this oracle evaluates (split
into row blocks only to bound memory: rows are independent).

The loss of the page's "Direct logits gradients" example, weighted squared
error, is written out here:  e = z - y,  w_ij = row_weight_i feature_weight_j,
loss = sum e^2 w,  d loss / d z = 2 e w.
"""
from __future__ import annotations

from typing import Callable

import numpy as np

_ROW_BLOCK_BYTES = 256 << 20


def weighted_mse_loss_and_grad(logits, target, row_weight, feature_weight):
    """(loss, d loss / d logits) of sum_ij (z_ij - y_ij)^2 r_i f_j, float64."""
    err = logits - target
    w = row_weight[:, None] * feature_weight[None, :]
    return float(np.sum(err * err * w)), 2.0 * err * w


def chunked_linear_loss(inputs, weight, loss_and_grad_fn: Callable, *row_args, row_block=None):
    """(loss, grad_inputs, grad_weight) in float64 for a row-additive loss.

    ``row_args`` are per-row arrays (leading dimension N) sliced with the rows,
    as the page describes for tensor arguments whose leading dimension is the
    batch; anything else must be bound into ``loss_and_grad_fn``."""
    n, h = inputs.shape
    vocab = weight.shape[0]
    rb = row_block or max(1, _ROW_BLOCK_BYTES // (8 * max(vocab, 1)))
    loss = 0.0
    gi = np.zeros((n, h))
    gw = np.zeros((vocab, h))
    for r0 in range(0, n, rb):
        r1 = min(n, r0 + rb)
        x = inputs[r0:r1]
        z = x @ weight.T
        part, g = loss_and_grad_fn(z, *(a[r0:r1] for a in row_args))
        loss += part
        gi[r0:r1] = g @ weight
        gw += g.T @ x
    return loss, gi, gw


def weighted_mse(inputs, weight, target, row_weight, feature_weight, row_block=None):
    """The generic path with the weighted squared error: (loss, grad_inputs, grad_weight)."""
    return chunked_linear_loss(
        inputs, weight,
        lambda z, y, r: weighted_mse_loss_and_grad(z, y, r, feature_weight),
        target, row_weight, row_block=row_block)
