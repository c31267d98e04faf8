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


def assert_num_correct(gpu_count, fwd):
    ambiguous = int((fwd.valid & (fwd.top2_gap < TOP2_GAP)).sum())
    assert abs(int(gpu_count) - fwd.num_correct) <= ambiguous, (
        f"num_correct {int(gpu_count)} vs oracle {fwd.num_correct} (ambiguous rows {ambiguous})")
