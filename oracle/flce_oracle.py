"""fp64 CPU oracle for fused linear cross-entropy.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's
``cpu_baseline`` leg may import this module.  The HIP library never calls it,
and it shares no code, tables or helpers with the HIP path.

What it computes is the plain definition of the loss, written out in float64
and evaluated row block by row block.  Rows are independent in the definition,
so splitting them into blocks changes nothing but memory use.  The sources:

* quack-kernels 0.2.0, ``quack/linear_cross_entropy.py``,
  ``linear_cross_entropy_func_ref``: the loss is ``F.linear(x, W, b)``
  followed by ``F.cross_entropy(..., ignore_index, reduction)``.
* fused-linear-ce README, "Usage" (signature) and "Algorithm": logits are
  ``hidden @ weight.T (+ bias)``, then bias / ``logit_scale`` / softcap are
  applied in that order; gradients for hidden, weight and bias are
  ``(p - onehot) @ weight``, ``(p - onehot).T @ hidden`` and the column sums.
* fused-linear-ce README, "Metrics for free": ``num_correct_tokens`` counts
  argmax == target and ``entropy_sum`` sums the softmax entropy in nats, both
  over non-ignored rows only.
* Chunked Linear Cross-Entropy (greyhound), "Usage": ``z_loss_multiplier``.
* Chunked Linear Loss (greyhound), "Reduction semantics": "mean" is one global
  mean over all valid tokens.

Readings taken where the pages are silent (each is listed with its reason in
the design notes):

1. z = softcap(logit_scale * (x.W^T + b)), the order the README lists.
2. softcap(v) = cap * tanh(v / cap); ``softcap`` None or <= 0 means off.
3. z-loss adds lambda * LSE_i^2 to each valid row's loss.
4. Metrics use the transformed logits z.
5. argmax ties resolve to the lowest vocabulary index.
6. "mean" with no valid row gives NaN loss, zero gradients and zero metrics.
7. "none" returns the per-row loss, 0 on ignored rows; its upstream gradient
   is a per-row vector.
8. LSE is computed for every row, ignored rows included.
9. A valid row's target must lie in [0, V); anything else raises.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

_ROW_BLOCK_BYTES = 256 << 20     # logits block size budget (float64)


def _row_block(n_rows: int, vocab: int) -> int:
    return int(max(1, min(n_rows, _ROW_BLOCK_BYTES // (8 * max(vocab, 1)))))


def _softcap_on(softcap: Optional[float]) -> bool:
    return softcap is not None and softcap > 0


def transform_logits(u: np.ndarray, logit_scale: float, softcap: Optional[float]) -> np.ndarray:
    """Bias already added to u; apply the scale, then the soft cap (readings 1, 2)."""
    v = logit_scale * u
    if _softcap_on(softcap):
        return softcap * np.tanh(v / softcap)
    return v


def _check_targets(targets: np.ndarray, vocab: int, ignore_index: int) -> np.ndarray:
    valid = targets != ignore_index
    bad = valid & ((targets < 0) | (targets >= vocab))
    if bad.any():
        raise ValueError(f"target out of range at rows {np.nonzero(bad)[0][:8].tolist()}")
    return valid


def _logits_block(x_blk, weight, bias, logit_scale, softcap):
    u = x_blk @ weight.T
    if bias is not None:
        u = u + bias[None, :]
    return transform_logits(u, logit_scale, softcap)


@dataclasses.dataclass
class ForwardResult:
    loss: np.ndarray            # scalar (sum | mean) or (N,) for "none"
    row_loss: np.ndarray        # (N,) per-row loss, 0 on ignored rows
    lse: np.ndarray             # (N,) log-sum-exp of z, every row
    argmax: np.ndarray          # (N,) lowest index of the row maximum
    top2_gap: np.ndarray        # (N,) largest minus second-largest z (0 on a tie, inf if V = 1)
    entropy: np.ndarray         # (N,) softmax entropy in nats, every row
    target_logit: np.ndarray    # (N,) z at the target, NaN on ignored rows
    valid: np.ndarray           # (N,) bool
    n_valid: int
    num_correct: int
    entropy_sum: float
    row_max: np.ndarray         # (N,) the row maximum of z (the value at argmax)


def forward(hidden, weight, bias, targets, *, logit_scale=1.0, softcap=None,
            z_loss=0.0, ignore_index=-100, reduction="mean",
            row_block: Optional[int] = None) -> ForwardResult:
    """Loss, LSE and metrics of ``softcap(scale * (hidden @ weight.T + bias))``.

    hidden (N,H), weight (V,H), bias (V,) or None: float64 arrays holding the
    exact values the device receives.  targets (N,) int64.
    """
    if reduction not in ("none", "sum", "mean"):
        raise ValueError(f"invalid reduction {reduction!r}")
    n, _ = hidden.shape
    vocab = weight.shape[0]
    valid = _check_targets(targets, vocab, ignore_index)
    lse = np.zeros(n)
    argmax = np.zeros(n, dtype=np.int64)
    gap = np.full(n, np.inf)
    ent = np.zeros(n)
    zt = np.full(n, np.nan)
    zmax = np.zeros(n)
    rb = row_block or _row_block(n, vocab)
    for r0 in range(0, n, rb):
        r1 = min(n, r0 + rb)
        z = _logits_block(hidden[r0:r1], weight, bias, logit_scale, softcap)
        m = z.max(axis=1)
        zmax[r0:r1] = m
        e = np.exp(z - m[:, None])
        s = e.sum(axis=1)
        lse[r0:r1] = m + np.log(s)
        p = e / s[:, None]
        ent[r0:r1] = lse[r0:r1] - (p * z).sum(axis=1)
        argmax[r0:r1] = np.argmax(z, axis=1)          # first maximum
        if vocab > 1:
            top2 = np.partition(z, vocab - 2, axis=1)[:, vocab - 2:]
            gap[r0:r1] = top2[:, 1] - top2[:, 0]
        rows = np.nonzero(valid[r0:r1])[0]
        zt[r0 + rows] = z[rows, targets[r0 + rows]]
    row_loss = np.where(valid, lse - np.where(valid, zt, 0.0) + z_loss * lse * lse, 0.0)
    n_valid = int(valid.sum())
    if reduction == "none":
        loss = row_loss.copy()
    elif reduction == "sum":
        loss = np.array(row_loss.sum())
    else:
        loss = np.array(row_loss.sum() / n_valid if n_valid else math.nan)
    num_correct = int((valid & (argmax == targets)).sum())
    entropy_sum = float(ent[valid].sum())
    return ForwardResult(loss, row_loss, lse, argmax, gap, ent, zt, valid, n_valid,
                         num_correct, entropy_sum, zmax)


def row_coefficients(targets, grad_loss, *, ignore_index=-100, reduction="mean"):
    """c_i: the upstream gradient reaching row i's loss (0 on ignored rows)."""
    valid = targets != ignore_index
    n_valid = int(valid.sum())
    g = np.asarray(grad_loss, dtype=np.float64)
    if reduction == "none":
        c = np.broadcast_to(g, targets.shape).astype(np.float64)
    elif reduction == "sum":
        c = np.full(targets.shape, float(g))
    elif reduction == "mean":
        c = np.full(targets.shape, float(g) / n_valid if n_valid else 0.0)
    else:
        raise ValueError(f"invalid reduction {reduction!r}")
    return np.where(valid, c, 0.0)


def logit_grad_block(z, lse, targets, coef, *, logit_scale=1.0, softcap=None,
                     z_loss=0.0, col_ids=None):
    """dLoss/du for a block of rows, u = x.W^T + b (the pre-transform logit).

    z (B, C) transformed logits of columns ``col_ids`` (all columns if None),
    lse (B,), targets (B,), coef (B,) from ``row_coefficients``.
    dLoss/dz = c * ((1 + 2*lambda*LSE) * p - onehot); the chain rule through
    the soft cap gives 1 - (z/cap)^2 and through the scale gives logit_scale.
    """
    p = np.exp(z - lse[:, None])
    dz = (1.0 + 2.0 * z_loss * lse)[:, None] * p
    cols = np.arange(z.shape[1]) if col_ids is None else np.asarray(col_ids)
    onehot = (cols[None, :] == targets[:, None])
    dz = coef[:, None] * (dz - onehot)
    if _softcap_on(softcap):
        dz = dz * (1.0 - (z / softcap) ** 2)
    return logit_scale * dz


def forward_backward(hidden, weight, bias, targets, grad_loss, *, logit_scale=1.0,
                     softcap=None, z_loss=0.0, ignore_index=-100, reduction="mean",
                     row_block: Optional[int] = None):
    """Forward result plus (grad_hidden, grad_weight, grad_bias), all float64."""
    fwd = forward(hidden, weight, bias, targets, logit_scale=logit_scale, softcap=softcap,
                  z_loss=z_loss, ignore_index=ignore_index, reduction=reduction,
                  row_block=row_block)
    coef = row_coefficients(targets, grad_loss, ignore_index=ignore_index, reduction=reduction)
    n, _ = hidden.shape
    vocab = weight.shape[0]
    gh = np.zeros_like(hidden)
    gw = np.zeros_like(weight)
    gb = np.zeros(vocab)
    rb = row_block or _row_block(n, vocab)
    for r0 in range(0, n, rb):
        r1 = min(n, r0 + rb)
        x = hidden[r0:r1]
        z = _logits_block(x, weight, bias, logit_scale, softcap)
        du = logit_grad_block(z, fwd.lse[r0:r1], targets[r0:r1], coef[r0:r1],
                              logit_scale=logit_scale, softcap=softcap, z_loss=z_loss)
        gh[r0:r1] = du @ weight
        gw += du.T @ x
        gb += du.sum(axis=0)
    return fwd, gh, gw, (gb if bias is not None else None)


def sampled_gradients(hidden, weight, bias, targets, grad_loss, lse, rows, vocab_ids, *,
                      logit_scale=1.0, softcap=None, z_loss=0.0, ignore_index=-100,
                      reduction="mean"):
    """grad_hidden at ``rows`` and grad_weight at ``vocab_ids``.

    ``lse`` must be the oracle's LSE for every row (grad_weight of one vocab
    row sums over all tokens).  Returns (grad_hidden[rows], grad_weight[vocab_ids]).
    """
    coef = row_coefficients(targets, grad_loss, ignore_index=ignore_index, reduction=reduction)
    rows = np.asarray(rows)
    vocab_ids = np.asarray(vocab_ids)
    z = _logits_block(hidden[rows], weight, bias, logit_scale, softcap)
    du = logit_grad_block(z, lse[rows], targets[rows], coef[rows], logit_scale=logit_scale,
                          softcap=softcap, z_loss=z_loss)
    gh = du @ weight
    n = hidden.shape[0]
    w_s = weight[vocab_ids]
    b_s = None if bias is None else bias[vocab_ids]
    gw = np.zeros((vocab_ids.size, hidden.shape[1]))
    rb = _row_block(n, vocab_ids.size)
    for r0 in range(0, n, rb):
        r1 = min(n, r0 + rb)
        zs = _logits_block(hidden[r0:r1], w_s, b_s, logit_scale, softcap)
        dus = logit_grad_block(zs, lse[r0:r1], targets[r0:r1], coef[r0:r1],
                               logit_scale=logit_scale, softcap=softcap, z_loss=z_loss,
                               col_ids=vocab_ids)
        gw += dus.T @ hidden[r0:r1]
    return gh, gw


def full_pass_with_bias_grad(hidden, weight, bias, targets, grad_loss, *, logit_scale=1.0,
                             softcap=None, z_loss=0.0, ignore_index=-100, reduction="mean",
                             row_block: Optional[int] = None, progress=None):
    """One pass over all rows: the forward result and the full grad_bias.

    Used at sizes where the full gradients are too costly: grad_bias needs
    every (row, vocab) probability but no extra contraction.
    """
    if reduction not in ("none", "sum", "mean"):
        raise ValueError(f"invalid reduction {reduction!r}")
    n, _ = hidden.shape
    vocab = weight.shape[0]
    valid = _check_targets(targets, vocab, ignore_index)
    coef = row_coefficients(targets, grad_loss, ignore_index=ignore_index, reduction=reduction)
    lse = np.zeros(n)
    argmax = np.zeros(n, dtype=np.int64)
    gap = np.full(n, np.inf)
    ent = np.zeros(n)
    zt = np.full(n, np.nan)
    zmax = np.zeros(n)
    gb = np.zeros(vocab)
    rb = row_block or _row_block(n, vocab)
    for r0 in range(0, n, rb):
        r1 = min(n, r0 + rb)
        z = _logits_block(hidden[r0:r1], weight, bias, logit_scale, softcap)
        m = z.max(axis=1)
        zmax[r0:r1] = m
        e = np.exp(z - m[:, None])
        s = e.sum(axis=1)
        lse_b = m + np.log(s)
        lse[r0:r1] = lse_b
        p = e / s[:, None]
        ent[r0:r1] = lse_b - (p * z).sum(axis=1)
        argmax[r0:r1] = np.argmax(z, axis=1)
        if vocab > 1:
            top2 = np.partition(z, vocab - 2, axis=1)[:, vocab - 2:]
            gap[r0:r1] = top2[:, 1] - top2[:, 0]
        rows = np.nonzero(valid[r0:r1])[0]
        zt[r0 + rows] = z[rows, targets[r0 + rows]]
        du = logit_grad_block(z, lse_b, targets[r0:r1], coef[r0:r1], logit_scale=logit_scale,
                              softcap=softcap, z_loss=z_loss)
        gb += du.sum(axis=0)
        if progress is not None:
            progress(r1, n)
    row_loss = np.where(valid, lse - np.where(valid, zt, 0.0) + z_loss * lse * lse, 0.0)
    n_valid = int(valid.sum())
    if reduction == "none":
        loss = row_loss.copy()
    elif reduction == "sum":
        loss = np.array(row_loss.sum())
    else:
        loss = np.array(row_loss.sum() / n_valid if n_valid else math.nan)
    num_correct = int((valid & (argmax == targets)).sum())
    fwd = ForwardResult(loss, row_loss, lse, argmax, gap, ent, zt, valid, n_valid,
                        num_correct, float(ent[valid].sum()), zmax)
    return fwd, gb
