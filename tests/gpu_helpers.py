"""Helpers shared by the GPU parity tests: device copies of seeded inputs and
the comparison rules (tolerances from the method's accuracy targets)."""
from __future__ import annotations

import numpy as np

import synth_inputs as si

# loss / LSE / entropy: relative error; gradients: max |err| <= GRAD_TOL * max |ref|
LOSS_RTOL = {"bf16": 2e-3, "f16": 2e-3, "f32": 1e-5}
GRAD_TOL = 1e-2
TOP2_GAP = 1e-3


def to_device(inp: dict, dtype: str, device="cuda"):
    import torch
    def dev(a):
        if a is None:
            return None
        if dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out = {k: dev(inp[k]) for k in ("hidden", "weight", "bias")}
    out["targets"] = torch.from_numpy(inp["targets"]).to(device)
    g = inp["grad_loss"]
    out["grad_loss"] = torch.from_numpy(np.atleast_1d(g).astype(np.float32)).to(device)
    return out


def widened(inp: dict, dtype: str):
    return (si.widen(inp["hidden"], dtype), si.widen(inp["weight"], dtype),
            si.widen(inp["bias"], dtype), inp["targets"])


def t2np(t):
    import torch
    if t is None:
        return None
    return t.detach().to(torch.float64).cpu().numpy()


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-30)))


def assert_loss_close(gpu, ref, dtype, what="loss"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if np.all(np.isnan(ref)):
        assert np.all(np.isnan(gpu)), f"{what}: expected NaN, got {gpu}"
        return
    tol = LOSS_RTOL[dtype]
    # elementwise: relative to |ref|, with an absolute floor for entries near zero
    scale = np.maximum(np.abs(ref), np.max(np.abs(ref)) * 1e-3 + 1e-30)
    err = np.max(np.abs(gpu - ref) / scale)
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.1e}"


def assert_grad_close(gpu, ref, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    if m == 0.0:
        assert err == 0.0, f"{what}: expected exact zeros, max |gpu| = {err:.3e}"
        return
    assert err <= GRAD_TOL * m, f"{what}: max err {err:.3e} > {GRAD_TOL:.0e} * max|ref| ({m:.3e})"


def ambiguous_rows(fwd) -> np.ndarray:
    """Valid rows whose argmax == target test can flip on rounding: the target's logit is
    within TOP2_GAP of the row maximum while another logit is too (top-2 gap < TOP2_GAP).
    A valid row outside this set has either its target as the unique maximum with margin
    (the count must include it) or its target more than TOP2_GAP below the maximum (it
    must not)."""
    zt = np.where(fwd.valid, np.nan_to_num(fwd.target_logit, nan=-np.inf), -np.inf)
    return fwd.valid & (fwd.row_max - zt < TOP2_GAP) & (fwd.top2_gap < TOP2_GAP)


def assert_num_correct(gpu_count, fwd, min_frac=None):
    """num_correct exact up to the ambiguous rows.  min_frac: also require (on the oracle
    side) that the oracle's count is at least that fraction of the valid rows and more
    than 100x the allowance, so that a kernel returning 0 or a wrong argmax merge fails."""
    amb = int(ambiguous_rows(fwd).sum())
    if min_frac is not None:
        assert fwd.num_correct >= min_frac * fwd.n_valid, (
            f"oracle num_correct {fwd.num_correct} < {min_frac} of {fwd.n_valid} valid rows")
        assert fwd.num_correct > 100 * amb, f"allowance {amb} too large for count {fwd.num_correct}"
    assert abs(int(gpu_count) - fwd.num_correct) <= amb, (
        f"num_correct {int(gpu_count)} vs oracle {fwd.num_correct} (ambiguous rows {amb})")
