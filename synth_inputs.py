"""Seeded synthetic inputs for the fused linear cross-entropy workloads.

This module only draws numbers: it holds none of the loss arithmetic, so that
both the fp64 oracle (``oracle/``) and the HIP path can be fed from it without
sharing any of the method's code.

Every array is drawn from numpy's PCG64 with a fixed seed.  A workload's seed
is split with ``SeedSequence.spawn`` into independent streams for hidden,
weight, bias, targets, the ignore mask and the upstream gradient, so changing
one recipe never moves another stream.

bf16 inputs are drawn as float32 normals and rounded to bfloat16 with
round-to-nearest-even; they are carried as their 16-bit patterns
(``np.uint16``).  fp16 inputs are the same normals rounded by numpy's
float32 -> float16 cast (also round-to-nearest-even) and carried as
``np.float16``.  ``widen`` turns any of them into the exact float64 values
that the oracle consumes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    hidden: int
    vocab: int
    dtype: str                      # "f32" | "bf16" | "f16"
    weight_std: float
    bias_std: Optional[float]       # None -> no bias
    logit_scale: float = 1.0
    softcap: Optional[float] = None
    z_loss: float = 0.0
    ignore_frac: float = 0.0
    reduction: str = "mean"         # "none" | "sum" | "mean"
    targets: str = "uniform"        # "uniform" | "zipf"
    zipf_s: float = 1.1
    grad_weight_dtype: Optional[str] = None   # None -> same as dtype
    return_metrics: bool = True
    seed: int = 0


# The five workloads: a tiny fp32 case, a 2k-token bf16 case, a Llama-2-like
# head, the 128k-vocabulary headline case and a 256k-vocabulary case.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 256, 128, 1024, "f32", 0.05, None,
                          reduction="sum", seed=0),
    "bf16_n2048_h1024_v32000": Workload(
        "bf16_n2048_h1024_v32000", 2048, 1024, 32000, "bf16", 0.02, None,
        ignore_frac=0.10, reduction="mean", seed=1),
    "bf16_n8192_h4096_v32000_zipf": Workload(
        "bf16_n8192_h4096_v32000_zipf", 8192, 4096, 32000, "bf16", 0.02, None,
        z_loss=1e-4, reduction="mean", targets="zipf", seed=2),
    "bf16_n8192_h4096_v128256": Workload(
        "bf16_n8192_h4096_v128256", 8192, 4096, 128256, "bf16", 0.02, 0.1,
        logit_scale=0.5, softcap=30.0, ignore_frac=0.05, reduction="sum", seed=3),
    "bf16_n16384_h2048_v256000": Workload(
        "bf16_n16384_h2048_v256000", 16384, 2048, 256000, "bf16", 0.02, None,
        reduction="none", grad_weight_dtype="f32", seed=4),
    # the headline case with fp16 inputs (fp16 is one of the input types the
    # fused-linear-ce signature lists), for the fp16 path's parity and timing
    "f16_n8192_h4096_v128256": Workload(
        "f16_n8192_h4096_v128256", 8192, 4096, 128256, "f16", 0.02, 0.1,
        logit_scale=0.5, softcap=30.0, ignore_frac=0.05, reduction="sum", seed=5),
}
HEADLINE = "bf16_n8192_h4096_v128256"


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step]
        bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
        flat_out[s:s + step] = ((u + bias) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def widen(arr: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact float64 copy of an input array (bf16 bit patterns, float16 or float32)."""
    if arr is None:
        return None
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return arr.astype(np.float64)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    out32 = np.empty(shape, dtype=np.float32)
    flat = out32.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        flat[s:s + n] = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        out32 *= np.float32(std)
    if dtype == "bf16":
        return round_to_bf16_bits(out32)
    if dtype == "f16":
        return out32.astype(np.float16)
    return out32


def _targets(rng: np.random.Generator, n: int, vocab: int, kind: str, zipf_s: float) -> np.ndarray:
    if kind == "uniform":
        return rng.integers(0, vocab, size=n, dtype=np.int64)
    if kind == "zipf":
        # finite Zipf on [0, vocab): P(k) proportional to (k+1)^-s, no permutation
        w = np.arange(1, vocab + 1, dtype=np.float64) ** (-zipf_s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = rng.random(n)
        return np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1).astype(np.int64)
    raise ValueError(kind)


def _round_to(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16_bits(x32)
    if dtype == "f16":
        return x32.astype(np.float16)
    return x32


def _plant(hidden: np.ndarray, weight: np.ndarray, t: np.ndarray, rows: np.ndarray, margin: float,
           dtype: str) -> None:
    """hidden[i] += margin * W[t_i] / |W[t_i]|^2 on the given rows, rounded back to the
    input type: the row's dot product with W[t_i] grows by about `margin` while its dot
    products with the other (nearly orthogonal) weight rows barely move.  Input
    construction only: the hidden rows of a batch whose targets are often its best match."""
    for r0 in range(0, rows.size, 4096):
        rr = rows[r0:r0 + 4096]
        w = widen(weight[t[rr]], dtype)
        x = widen(hidden[rr], dtype)
        x += margin * w / np.maximum((w * w).sum(axis=1, keepdims=True), 1e-30)
        hidden[rr] = _round_to(x, dtype)


def make_inputs(n_tokens: int, hidden: int, vocab: int, *, dtype: str = "bf16",
                weight_std: float = 0.02, hidden_std: float = 1.0,
                bias_std: Optional[float] = None, targets: str = "uniform",
                zipf_s: float = 1.1, ignore_frac: float = 0.0,
                reduction: str = "mean", seed: int = 0, plant_frac: float = 0.0,
                plant_margin: float = 8.0) -> dict:
    """Draw one problem.  Returns numpy arrays:

    hidden (N,H), weight (V,H), bias (V,) or None -- uint16 bf16 patterns, float16 or float32;
    targets (N,) int64 with exactly floor(ignore_frac*N) entries set to -100;
    grad_loss: float32 scalar 1.0 for sum/mean, (N,) N(0,1) for "none".

    plant_frac > 0: a seeded floor(plant_frac*N) of the rows get a component
    along their target's weight row (``_plant``, `plant_margin` in units of the
    raw dot product), so that the target is usually the row's largest logit and
    the argmax count is far from zero.  The other streams are unchanged.
    """
    ss = np.random.SeedSequence(seed)
    s_h, s_w, s_b, s_t, s_i, s_g, s_p = ss.spawn(7)
    out = {
        "hidden": _normal(np.random.Generator(np.random.PCG64(s_h)), (n_tokens, hidden), hidden_std, dtype),
        "weight": _normal(np.random.Generator(np.random.PCG64(s_w)), (vocab, hidden), weight_std, dtype),
        "bias": (None if bias_std is None else
                 _normal(np.random.Generator(np.random.PCG64(s_b)), (vocab,), bias_std, dtype)),
    }
    t = _targets(np.random.Generator(np.random.PCG64(s_t)), n_tokens, vocab, targets, zipf_s)
    n_plant = int(np.floor(plant_frac * n_tokens))
    if n_plant:
        rows = np.sort(np.random.Generator(np.random.PCG64(s_p)).permutation(n_tokens)[:n_plant])
        _plant(out["hidden"], out["weight"], t, rows, plant_margin, dtype)
    n_ign = int(np.floor(ignore_frac * n_tokens))
    if n_ign:
        perm = np.random.Generator(np.random.PCG64(s_i)).permutation(n_tokens)
        t[perm[:n_ign]] = IGNORE_INDEX
    out["targets"] = t
    if reduction == "none":
        out["grad_loss"] = np.random.Generator(np.random.PCG64(s_g)).standard_normal(
            n_tokens, dtype=np.float32)
    else:
        out["grad_loss"] = np.array(1.0, dtype=np.float32)
    return out


def make_workload_inputs(wl: Workload) -> dict:
    return make_inputs(wl.n_tokens, wl.hidden, wl.vocab, dtype=wl.dtype,
                       weight_std=wl.weight_std, bias_std=wl.bias_std,
                       targets=wl.targets, zipf_s=wl.zipf_s,
                       ignore_frac=wl.ignore_frac, reduction=wl.reduction,
                       seed=wl.seed)


def make_wmse_inputs(n_tokens: int, hidden: int, vocab: int, *, dtype: str = "bf16",
                     weight_std: float = 0.02, hidden_std: float = 1.0, seed: int = 0) -> dict:
    """Inputs of the weighted squared error through the generic chunked loss:
    hidden (N,H) and weight (V,H) as in ``make_inputs``; target (N,V) float32
    N(0,1); row_weight (N,) and feature_weight (V,) float32 uniform in [0.5, 1.5)."""
    ss = np.random.SeedSequence(seed)
    s_h, s_w, s_y, s_r, s_f = ss.spawn(5)
    target = np.empty((n_tokens, vocab), dtype=np.float32)
    flat = target.reshape(-1)
    g = np.random.Generator(np.random.PCG64(s_y))
    step = 1 << 24
    for s0 in range(0, flat.size, step):
        k = min(step, flat.size - s0)
        flat[s0:s0 + k] = g.standard_normal(k, dtype=np.float32)
    return {
        "hidden": _normal(np.random.Generator(np.random.PCG64(s_h)), (n_tokens, hidden), hidden_std, dtype),
        "weight": _normal(np.random.Generator(np.random.PCG64(s_w)), (vocab, hidden), weight_std, dtype),
        "target": target,
        "row_weight": np.random.Generator(np.random.PCG64(s_r)).uniform(0.5, 1.5, n_tokens).astype(np.float32),
        "feature_weight": np.random.Generator(np.random.PCG64(s_f)).uniform(0.5, 1.5, vocab).astype(np.float32),
    }


# The weighted squared error through the generic chunked loss at the headline
# projection shape (N=8192, H=4096, V=128256): (n_tokens, hidden, vocab, dtype, weight_std, seed).
WMSE_WORKLOADS = {
    "wmse_bf16_n8192_h4096_v128256": (8192, 4096, 128256, "bf16", 0.02, 6),
}
