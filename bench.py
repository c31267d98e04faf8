"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path split|both|fused]
                    [--vocab-chunk C] [--block-rows R] [--grad-weight-accum fp32|weight] [--no-cpu-baseline]
                    [--power-seconds S]

One step is a full forward + backward (loss, LSE, metrics, grad_hidden,
grad_weight, grad_bias) on the headline workload: N=8192 tokens, H=4096,
V=128256, bf16, bias, logit_scale 0.5, softcap 30, 5% ignored targets,
reduction "sum", through flce_forward then flce_backward (the backward
recomputes the logit tiles: 8*N*H*V flop per step, the metric's count).
Inputs are seeded synthetic data already resident in device memory; outputs
and workspaces are allocated before timing.

Prints one JSON line.  `value` is tokens/s of the whole step (wall clock over
the K timed steps, bracketed by device synchronizations); `tflops` counts
8*N*H*V per step.  Inside the timed steps the two calls go through
flce_forward_timed / flce_backward_timed, which record HIP events on the
calls' stream around every matrix-core launch: `kernels` gives each kernel's
time per step, and `roofline` reports the one with the largest share.
`--path both` also times flce_forward_backward (one pass over row blocks, no
recompute, 6*N*H*V flop) as the side object `one_pass`.  `cpu_baseline` times
the fp64 CPU oracle on a bounded slice of the same workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth_inputs as si  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 (and fp16) MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "fwd+bwd tokens/s and TFLOP/s (8NHV) vs bf16 MFMA peak, N=8192 H=4096 V=128k"
CSRC = os.path.join(ROOT, "linear_cross_entropy_tiled_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def _code_only(text: str) -> str:
    """The source without its comments and with whitespace runs collapsed, so
    that editing a comment does not count as a change of the kernels."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the HIP sources' code (comments and layout ignored); a traffic
    figure is only reported for the kernels it was measured on."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(CSRC, "*.hip"))):
        h.update(os.path.basename(f).encode())
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel`, from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None if there is none or it is stale."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash() or kv.get("kernel") != kernel:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _device_info(torch):
    """Name, compute units and architecture of the GPU as the runtime reports them (the peak assumes 256 CUs)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "compute_units": p.multi_processor_count,
            "arch": getattr(p, "gcnArchName", ""), "memory_gib": round(p.total_memory / 2**30, 1)}


def _to_dev(inp, dtype):
    import torch
    def dev(a):
        if a is None:
            return None
        if dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    d = {k: dev(inp[k]) for k in ("hidden", "weight", "bias")}
    d["targets"] = torch.from_numpy(inp["targets"]).cuda()
    d["grad_loss"] = torch.from_numpy(np.atleast_1d(inp["grad_loss"]).astype(np.float32)).cuda()
    return d


def cpu_baseline(inp, wl, rows: int):
    """The fp64 oracle (as is) on the first `rows` tokens of the workload."""
    import oracle
    x = si.widen(inp["hidden"][:rows], wl.dtype)
    w = si.widen(inp["weight"], wl.dtype)
    b = si.widen(inp["bias"], wl.dtype)
    t = inp["targets"][:rows]
    g = inp["grad_loss"][:rows] if wl.reduction == "none" else inp["grad_loss"]
    t0 = time.perf_counter()
    oracle.forward_backward(x, w, b, t, np.asarray(g, dtype=np.float64), logit_scale=wl.logit_scale,
                            softcap=wl.softcap, z_loss=wl.z_loss, reduction=wl.reduction)
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": rows / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle forward+backward of the first {rows} of {wl.n_tokens} tokens "
                      f"against the full {wl.vocab}-row weight ({dt:.1f} s)",
            "seconds": dt, "gflops": 6.0 * rows * wl.hidden * wl.vocab / dt / 1e9}


class PowerSampler:
    """Read-only board telemetry (socket power, graphics clock) through amdsmi, sampled in a
    background thread.  The readings refresh about once a second, so it runs over a window of
    several seconds of steady work, outside the timed steps."""

    def __init__(self, period_s: float = 0.05):
        import threading
        import amdsmi
        self.amdsmi = amdsmi
        amdsmi.amdsmi_init()
        self.h = amdsmi.amdsmi_get_processor_handles()[0]
        self.period = period_s
        self.samples = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        a = self.amdsmi
        while not self.stop.is_set():
            try:
                p = a.amdsmi_get_power_info(self.h)
                c = a.amdsmi_get_clock_info(self.h, a.AmdSmiClkType.GFX)
                self.samples.append((time.perf_counter(), float(p["current_socket_power"]), float(c["clk"])))
            except Exception:
                pass
            self.stop.wait(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join()

    def summary(self, skip_s: float = 1.5):
        a = self.amdsmi
        try:
            cap = float(a.amdsmi_get_power_cap_info(self.h)["power_cap"]) / 1e6
        except Exception:
            cap = None
        a.amdsmi_shut_down()
        if not self.samples:
            return None
        t0 = self.samples[0][0]
        s = [(p, c) for t, p, c in self.samples if t - t0 >= skip_s] or [(p, c) for _, p, c in self.samples]
        return {"socket_power_w_mean": float(np.mean([p for p, _ in s])), "socket_power_w_max": max(p for p, _ in s),
                "gfx_clock_mhz_mean": float(np.mean([c for _, c in s])), "power_cap_w": cap, "samples": len(s),
                "note": "amdsmi telemetry over extra untimed steps after the timed ones (first 1.5 s dropped)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=si.HEADLINE, choices=sorted(si.WORKLOADS) + sorted(si.WMSE_WORKLOADS))
    ap.add_argument("--path", choices=("split", "both", "fused"), default="split",
                    help="split (default): flce_forward then flce_backward (the backward recomputes the logit "
                         "tiles), the measured step; both: also time flce_forward_backward (one pass: gradients "
                         "from each row block's stored logits, 6NHV) as the side object one_pass; fused: only "
                         "the one-pass step")
    ap.add_argument("--vocab-chunk", type=int, default=0,
                    help="flce_backward: vocabulary rows per logit-gradient chunk (multiple of 256; 0 = the "
                         "library's choice)")
    ap.add_argument("--block-rows", type=int, default=0,
                    help="rows per block of flce_forward_backward (a multiple of 256; 0 = the library's choice)")
    ap.add_argument("--grad-weight-accum", choices=("fp32", "weight"), default="fp32",
                    help="flce_forward_backward: sum grad_weight over the row blocks in fp32 (default) or in its "
                         "own dtype")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, copy this many MiB device-to-device once (counter calibration)")
    ap.add_argument("--power-seconds", type=float, default=0.0,
                    help="after the timed steps, run steps for this many more seconds while sampling socket power "
                         "and graphics clock (amdsmi telemetry, read only); reported as `power`")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_cross_entropy_tiled_amd as flce

    flce.load()
    if args.workload in si.WMSE_WORKLOADS:
        return run_wmse(args, torch, flce)
    wl = si.WORKLOADS[args.workload]
    inp = si.make_workload_inputs(wl)
    d = _to_dev(inp, wl.dtype)
    n, h, v = wl.n_tokens, wl.hidden, wl.vocab
    opts = dict(logit_scale=wl.logit_scale, softcap=wl.softcap, z_loss=wl.z_loss,
                ignore_index=si.IGNORE_INDEX, reduction=wl.reduction)
    pf = flce.make_params(n, h, v, dtype=wl.dtype, grad_weight_dtype=wl.grad_weight_dtype,
                          grad_weight_accum_dtype=args.grad_weight_accum, vocab_chunk=args.vocab_chunk, **opts)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    loss = torch.empty(n if wl.reduction == "none" else 1, dtype=torch.float32, device="cuda")
    lse = torch.empty(n, dtype=torch.float32, device="cuda")
    nc = torch.empty(1, dtype=torch.int64, device="cuda")
    ent = torch.empty(1, dtype=torch.float32, device="cuda")
    gh = torch.empty((n, h), dtype=tdt[wl.dtype], device="cuda")
    gw = torch.empty((v, h), dtype=tdt[wl.grad_weight_dtype or wl.dtype], device="cuda")
    gb = torch.empty(v, dtype=tdt[wl.dtype], device="cuda") if d["bias"] is not None else None
    gl = d["grad_loss"] if wl.reduction == "none" else d["grad_loss"][:1]
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    flop8 = 8.0 * n * h * v
    peak = PEAK_BF16_TFLOPS if wl.dtype in ("bf16", "f16") else PEAK_F32_TFLOPS

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def time_fused():
        ws = torch.empty(flce.flce_forward_backward_workspace_size(pf, args.block_rows), dtype=torch.uint8,
                         device="cuda")

        def step():
            rc = flce.flce_forward_backward(pf, args.block_rows, P(d["hidden"]), P(d["weight"]), P(d["bias"]),
                                            P(d["targets"]), P(gl), P(loss), P(lse), P(nc), P(ent), P(gh), P(gw),
                                            P(gb), P(ws), ws.numel(), sh)
            if rc:
                raise flce.FlceError(rc, "flce_forward_backward")

        torch.cuda.reset_peak_memory_stats()
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) / args.steps * 1e3
        mem = torch.cuda.max_memory_allocated() / 2**30
        del ws
        torch.cuda.empty_cache()
        # the one-pass step executes 6NHV: no recompute
        flop6 = 0.75 * flop8
        return {"path": "flce_forward_backward (one pass over row blocks, no recompute: 6NHV executed)",
                "ms_per_step": step_ms, "value": n / (step_ms * 1e-3), "unit": "tokens/s", "peak_mem_gib": mem,
                "tflops_executed": flop6 / (step_ms * 1e-3) / 1e12,
                "frac_of_peak_executed": flop6 / (step_ms * 1e-3) / 1e12 / peak}

    def time_split():
        ws_f = torch.empty(flce.flce_workspace_size(pf, flce.FLCE_PASS_FORWARD), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(flce.flce_workspace_size(pf, flce.FLCE_PASS_BACKWARD), dtype=torch.uint8, device="cuda")
        # one event pair per matrix-core launch: the forward tile kernel, then 3 per vocabulary
        # chunk; the first warm-up step counts them (at most one chunk per 256 vocabulary rows)
        probe = flce.LaunchTimer(capacity=1 + 3 * ((v + 255) // 256), stream=stream)

        def fwd(t):
            rc = flce.flce_forward_timed(pf, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]),
                                         P(loss), P(lse), P(nc), P(ent), P(ws_f), ws_f.numel(), sh, t)
            if rc:
                raise flce.FlceError(rc, "flce_forward")

        def bwd(t):
            rc = flce.flce_backward_timed(pf, P(d["hidden"]), P(d["weight"]), P(d["bias"]), P(d["targets"]),
                                          P(lse), P(gl), P(gh), P(gw), P(gb), P(ws_b), ws_b.numel(), sh, t)
            if rc:
                raise flce.FlceError(rc, "flce_backward")

        torch.cuda.reset_peak_memory_stats()
        for i in range(max(args.warmup, 1)):
            fwd(probe.c if i == 0 else None)
            bwd(probe.c if i == 0 else None)
        torch.cuda.synchronize()
        timer = flce.LaunchTimer(capacity=args.steps * probe.c.count, stream=stream)
        del probe
        # HIP events on the stream the kernels run on bracket each call and each launch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        timer.reset()
        t0 = time.perf_counter()
        for e0, e1, e2 in ev:
            e0.record(stream)
            fwd(timer.c)
            e1.record(stream)
            bwd(timer.c)
            e2.record(stream)
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) / args.steps * 1e3
        fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
        bwd_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
        launches = timer.durations()
        power = None
        if args.power_seconds > 0:
            try:
                sampler = PowerSampler()
            except Exception as e:   # no telemetry on this machine
                power = {"error": f"{type(e).__name__}: {e}"}
            else:
                with sampler:
                    t1 = time.perf_counter()
                    while time.perf_counter() - t1 < args.power_seconds:
                        for _ in range(4):
                            fwd(None)
                            bwd(None)
                        torch.cuda.synchronize()
                power = sampler.summary()
        mem = torch.cuda.max_memory_allocated() / 2**30
        del ws_f, ws_b
        torch.cuda.empty_cache()
        # every kernel of the four does 2NHV per step in total (the chunk kernels in
        # launches of 2*N*H*(rows of the chunk))
        kernels = {}
        for name, ms in launches.items():
            per_step = float(np.sum(ms)) / args.steps
            kernels[name] = {"launches_per_step": len(ms) // args.steps, "ms_per_step": per_step,
                             "mean_launch_ms": float(np.mean(ms)),
                             "tflops": 0.25 * flop8 / (per_step * 1e-3) / 1e12,
                             "share_of_step": per_step / step_ms}
        return {"ms_per_step": step_ms, "value": n / (step_ms * 1e-3), "peak_mem_gib": mem,
                "tflops_8nhv": flop8 / (step_ms * 1e-3) / 1e12, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
                "fwd_tflops": 0.25 * flop8 / (fwd_ms * 1e-3) / 1e12,
                "bwd_tflops": 0.75 * flop8 / (bwd_ms * 1e-3) / 1e12, "kernels": kernels, "power": power}

    split = time_split() if args.path in ("both", "split") else None
    fused = time_fused() if args.path in ("both", "fused") else None
    plan_chunks = None
    if split is not None:
        lk = split["kernels"].get("bwd_dlogits_kernel")
        plan_chunks = lk["launches_per_step"] if lk else None
    cfg = {"workload": wl.name, "n_tokens": n, "hidden": h, "vocab": v, "bias": wl.bias_std is not None,
           "logit_scale": wl.logit_scale, "softcap": wl.softcap, "z_loss": wl.z_loss,
           "ignore_frac": wl.ignore_frac, "reduction": wl.reduction,
           "grad_weight_dtype": wl.grad_weight_dtype or wl.dtype,
           "vocab_chunk": args.vocab_chunk or "library choice", "vocab_chunks_per_step": plan_chunks,
           "path": ("flce_forward + flce_backward (the backward recomputes the logit tiles)" if split is not None
                    else "flce_forward_backward (one pass, no recompute)")}
    out = {
        "metric": METRIC,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": cfg,
        "device": _device_info(torch),
        "kernel_source_hash": kernel_source_hash(),
    }
    if split is not None:
        out.update({
            "value": split["value"],
            "ms_per_step": split["ms_per_step"],
            # the metric's count: 8NHV flop per step (forward logits, recomputed logits, two contractions)
            "tflops": split["tflops_8nhv"],
            "frac_of_peak": split["tflops_8nhv"] / peak,
            "peak_mem_gib": split["peak_mem_gib"],
            "fwd_ms": split["fwd_ms"], "bwd_ms": split["bwd_ms"],
            "fwd_tflops": split["fwd_tflops"], "bwd_tflops": split["bwd_tflops"],
            "kernels": split["kernels"],
        })
        if split["power"] is not None:
            out["power"] = split["power"]
        # the kernel with the largest share of the step, its launches timed with HIP events on
        # the stream they run on; achieved = its algorithmic flops per step (2NHV) over its time
        # per step, i.e. per-launch flops over mean launch duration
        name, k = max(split["kernels"].items(), key=lambda kv: kv[1]["ms_per_step"])
        out["roofline"] = {"bound": "mfma", "kernel": name, "achieved": k["tflops"], "peak": peak,
                           "unit": "TFLOP/s", "frac": k["tflops"] / peak,
                           "traffic": measured_traffic(name, wl.name),
                           "launches_per_step": k["launches_per_step"], "mean_launch_ms": k["mean_launch_ms"],
                           "share_of_step": k["share_of_step"]}
    else:
        out.update({"value": fused["value"], "ms_per_step": fused["ms_per_step"],
                    "tflops_executed": fused["tflops_executed"],
                    "frac_of_peak_executed": fused["frac_of_peak_executed"], "peak_mem_gib": fused["peak_mem_gib"]})
    if fused is not None and split is not None:
        out["one_pass"] = fused
    if not args.no_cpu_baseline:
        del d
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(inp, wl, min(args.cpu_rows, n))
    print(json.dumps(out), flush=True)


def run_wmse(args, torch, flce):
    """One step = one flce_chunked_linear_loss call with the built-in weighted
    squared error: block logits (2NHV), the loss kernel, grad_inputs (2NHV)
    and grad_weight (2NHV); 6NHV flop."""
    import ctypes
    name = args.workload
    n, h, v, dtype, wstd, seed = si.WMSE_WORKLOADS[name]
    inp = si.make_wmse_inputs(n, h, v, dtype=dtype, weight_std=wstd, seed=seed)
    d = _to_dev({k: inp[k] for k in ("hidden", "weight")} | {"bias": None, "targets": np.zeros(1, np.int64),
                                                           "grad_loss": np.float32(1.0)}, dtype)
    y = torch.from_numpy(inp["target"]).cuda()
    r = torch.from_numpy(inp["row_weight"]).cuda()
    f = torch.from_numpy(inp["feature_weight"]).cuda()
    p = flce.make_chunked_params(n, h, v, dtype=dtype)
    ws = torch.empty(flce.flce_chunked_workspace_size(p), dtype=torch.uint8, device="cuda")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    gi = torch.empty((n, h), dtype=tdt[dtype], device="cuda")
    gw = torch.empty((v, h), dtype=tdt[dtype], device="cuda")
    row_loss = torch.empty(n, dtype=torch.float32, device="cuda")
    a = flce.flce_wmse_args(y.data_ptr(), y.stride(0), r.data_ptr(), f.data_ptr(), row_loss.data_ptr())
    user = ctypes.cast(ctypes.pointer(a), ctypes.c_void_p)
    fn = flce.weighted_mse_chunk_fn()
    stream = torch.cuda.current_stream()

    def step():
        rc = flce.flce_chunked_linear_loss(p, d["hidden"].data_ptr(), d["weight"].data_ptr(), fn, user,
                                           loss.data_ptr(), gi.data_ptr(), gw.data_ptr(), ws.data_ptr(),
                                           ws.numel(), stream.cuda_stream)
        if rc:
            raise flce.FlceError(rc, "flce_chunked_linear_loss")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall / args.steps * 1e3
    ev_ms = float(np.mean([x.elapsed_time(z) for x, z in ev]))
    tflops = 6.0 * n * h * v / (step_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if dtype in ("bf16", "f16") else PEAK_F32_TFLOPS
    out = {
        "metric": "generic chunked linear loss (weighted squared error) tokens/s and TFLOP/s (6NHV)",
        "value": n / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": name, "n_tokens": n, "hidden": h, "vocab": v, "loss": "weighted squared error",
                   "rows_per_block": int(p.chunk_rows) or "library choice", "grad_weight_accum_dtype": "fp32"},
        "tflops": tflops,
        "frac_of_peak": tflops / peak,
        "event_ms_per_step": ev_ms,
        "peak_mem_gib": torch.cuda.max_memory_allocated() / 2**30,
        "device": _device_info(torch),
        "roofline": {"bound": "mfma", "kernel": "whole step (block logits + two contractions, 6NHV)",
                     "achieved": 6.0 * n * h * v / (ev_ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
                     "frac": 6.0 * n * h * v / (ev_ms * 1e-3) / 1e12 / peak, "traffic": None},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = min(args.cpu_rows, n) // 4
        x = si.widen(inp["hidden"][:rows], dtype)
        w = si.widen(inp["weight"], dtype)
        t1 = time.perf_counter()
        oracle.weighted_mse(x, w, inp["target"][:rows].astype(np.float64),
                            inp["row_weight"][:rows].astype(np.float64), inp["feature_weight"].astype(np.float64))
        dt = time.perf_counter() - t1
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count()
        out["cpu_baseline"] = {"value": rows / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                               "sample": f"fp64 oracle weighted squared error of the first {rows} of {n} tokens "
                                         f"against the full {v}-row weight ({dt:.1f} s)", "seconds": dt}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
