#!/usr/bin/env python3
"""Benchmark of the fused RNN operator on one MI355X.

One step = one full training pass of the hot path on one batch of synthetic
input: rnn_forward_training + rnn_backward_data + rnn_backward_weights
(hoisted input GEMM, persistent recurrent sweep with fused gates, reserve
fill, BPTT sweep, dX GEMM, dW GEMMs).  Workload: single-layer unidirectional
LSTM at the Deep Speech 2 shape (T=300, B=20, input=800, hidden=800), bf16
weights with fp32 state and accumulation (headline); the fp32-weight variant
is reported next to it.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  GFLOP/s counts GEMM flops only (2*M*N*K): forward
2*T*B*G*H*(I+H), training step three times that.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "fused RNN train-step GFLOP/s + fwd ms at DS2 shape (T300 B20 H800); % MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, MI355X
HBM_GBS = 8000.0


def flops(mode, T, B, I, H, L, D):
    G = {"rnn_tanh": 1, "lstm": 4, "gru": 3, "gru_tf": 3, "gru_paper": 3}[mode]
    f = 0
    for l in range(L):
        I_l = I if l == 0 else D * H
        f += D * 2 * T * B * G * H * (I_l + H)
    return f


class Runner:
    def __init__(self, w, torch, R, synth, dropout=0.0):
        self.torch, self.R = torch, R
        self.w = w
        self.dropout, self.seed = dropout, 0
        case = synth.make_workload(w)
        T, B, I, H, L, D = w.T, w.B, w.input_size, w.hidden, w.layers, w.dirs
        self.T, self.B = T, B
        self.h = R.rnn_create(w.mode, L, D, I, H, w.wtype)
        if dropout > 0.0:   # before the workspace is sized
            R.rnn_set_dropout(self.h, dropout, 0)
        dev = "cuda"
        f32 = torch.float32
        t = lambda a: None if a is None else torch.as_tensor(a, dtype=torch.float64).to(f32).to(dev)
        self.W = R.pack_weights(self.h, case["params"], dev)
        self.x, self.h0, self.c0 = t(case["x"]), t(case["h0"]), t(case["c0"])
        self.dy = t(case["dy"])
        self.y = torch.empty((T, B, D * H), device=dev)
        self.hy = torch.empty((L * D, B, H), device=dev)
        self.cy = torch.empty((L * D, B, H), device=dev) if w.mode == "lstm" else None
        self.dx = torch.empty((T, B, I), device=dev)
        self.dh0 = torch.empty((L * D, B, H), device=dev)
        self.dc0 = torch.empty((L * D, B, H), device=dev) if w.mode == "lstm" else None
        self.dW = torch.empty((R.rnn_weights_size(self.h, 1) // 4,), device=dev)
        self.ws = torch.empty(R.rnn_workspace_size(self.h, T, B, 1), dtype=torch.uint8, device=dev)
        self.ws_inf = torch.empty(R.rnn_workspace_size(self.h, T, B, 0), dtype=torch.uint8, device=dev)

    def train_step(self):
        R, T, B = self.R, self.T, self.B
        if self.dropout > 0.0:   # fresh masks every step
            self.seed += 1
            R.rnn_set_dropout(self.h, self.dropout, self.seed)
        R.rnn_forward_training(self.h, T, B, self.x, self.h0, self.c0, self.W, self.y, self.hy,
                               self.cy, self.ws)
        R.rnn_backward_data(self.h, T, B, self.y, self.dy, None, None, self.W, self.h0, self.c0,
                            self.dx, self.dh0, self.dc0, self.ws)
        R.rnn_backward_weights(self.h, T, B, self.x, self.h0, self.y, self.ws, self.dW)

    def fwd(self):
        self.R.rnn_forward_inference(self.h, self.T, self.B, self.x, self.h0, self.c0, self.W,
                                     self.y, self.hy, self.cy, self.ws_inf)

    def graph_timed(self, steps, warmup):
        """The same training step captured once into a HIP graph on this
        stream and replayed: what a caller that captures its step sees (the
        library allocates, memsets and synchronises nothing inside its calls).
        Mean ms per replay over `steps` replays."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.train_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.train_step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def timed(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        times = []
        s = torch.cuda.current_stream()
        t0 = time.perf_counter()
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            fn()
            b.record(s)
            times.append((a, b))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [a.elapsed_time(b) for a, b in times]
        return ms, wall


def cpu_baseline(w, synth, min_seconds):
    """The fp64 oracle on the host cores: full training steps of the same
    workload (forward + backward through time + weight gradients), repeated
    until at least `min_seconds` of CPU work have been timed."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import rnn_oracle as orc
    case = synth.make_workload(w)
    D = w.dirs
    # the library's GRU flavour modes are oracle GRU variants
    variant = {"gru_tf": "tf", "gru_paper": "paper"}.get(w.mode, "pytorch")
    mode = "gru" if variant != "pytorch" else w.mode
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        _, _, _, cache = orc.forward(mode, case["x"], case["params"], h0=case["h0"],
                                     c0=case["c0"], num_dirs=D, gru_variant=variant, keep=True)
        orc.backward(mode, case["params"], cache, case["dy"], num_dirs=D)
        dt += time.perf_counter() - t0
        reps += 1
    f = reps * 3 * flops(w.mode, w.T, w.B, w.input_size, w.hidden, w.layers, D)
    cores = None
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 0) for i in threadpool_info()), default=None)
    except Exception:
        pass
    return {"value": round(f / dt / 1e9, 3), "unit": "GFLOP/s", "cores": cores or os.cpu_count(),
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{w.name}: {reps} full training step(s) (T={w.T}) in fp64 on the host, "
                      f"forward + backward through time + weight gradients, {dt:.1f} s"}


def source_hash():
    """sha256[:16] over every native source of the library (kernels, their
    headers and the host planner, which decides grids and layouts): a
    counter figure taken under another hash is stale."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(root, "layer_rnn_forward_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the library sources changed since it was taken."""
    import glob
    root = os.path.dirname(os.path.abspath(__file__))
    h = source_hash()
    for path in glob.glob(os.path.join(root, "profiles", "traffic_*.txt")):
        for line in open(path):
            parts = line.split()
            if len(parts) == 4 and parts[0] == "TRAFFIC" and parts[1] == h and parts[2] == kernel:
                return int(parts[3])
    return None


def copy_calibration(torch, mib=1024, reps=3):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "reps": reps}))


def mfma_peak(torch, R, kind, reps=3):
    """Measured dense MFMA throughput (TFLOP/s) of this device for one MFMA
    instruction: the library's throughput probe on two workgroups per CU,
    timed with events."""
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    flop1, A, K, iters = {"f32_16x16x4": (8192, 32, 16, 2000), "bf16_16x16x32": (16384, 32, 32, 10000),
                          "bf16_32x32x16": (32768, 128, 16, 5000)}[kind]
    out = torch.empty(blocks * 256, device="cuda")
    R.rnn_mfma_peak_probe(kind, blocks, iters // 10, out)   # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        R.rnn_mfma_peak_probe(kind, blocks, iters, out)
    e1.record()
    torch.cuda.synchronize()
    assert float(out[0]) == A * iters * K / 512.0, "MFMA probe result"
    flop = reps * blocks * 4 * iters * 8 * flop1
    return flop / (e0.elapsed_time(e1) * 1e-3) / 1e12


def blas_reference(torch, w, reps=50):
    """Context for the GEMM rows: the vendor BLAS (hipBLASLt through torch.mm,
    bf16 operands, bf16 output, operands in the same K-contiguous layout as
    this library's) on the three time-parallel products of the workload.
    Not part of the operator; reported only with --blas-reference."""
    G = {"rnn_tanh": 1, "lstm": 4, "gru": 3, "gru_tf": 3, "gru_paper": 3}[w.mode]
    TB, N, I = w.T * w.B, w.dirs * G * w.hidden, w.input_size
    shapes = {"gemm_input": (TB, N, I), "gemm_dx": (TB, I, N), "gemm_dw (one of dW_ih, dW_hh)": (N, I, TB)}
    out = {}
    for name, (M, Nn, K) in shapes.items():
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(Nn, K, device="cuda", dtype=torch.bfloat16)
        for _ in range(5):
            torch.mm(a, b.t())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.mm(a, b.t())
        e1.record()
        torch.cuda.synchronize()
        us = 1000.0 * e0.elapsed_time(e1) / reps
        tf = 2.0 * M * Nn * K / (us * 1e-6) / 1e12
        out[name] = {"M": M, "N": Nn, "K": K, "avg_us": round(us, 2), "TFLOPs": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}
    return out


GATES = {"rnn_tanh": 1, "lstm": 4, "gru": 3, "gru_tf": 3, "gru_paper": 3}

# stacked and GRU workloads reported next to the headline (one GPU, same step)
SECONDARY = ("gru_ds2_f32", "lstm_ds2_l5_bi_bf16", "gru_ds2_l5_bi_bf16", "tanh_ds2_l5_bi_bf16",
             "lstm_ds2_l5_uni_bf16")


def kernel_flops(w):
    """Algorithmic GEMM flops per training step of each kernel kind (2*M*N*K
    summed over layers; the bias-gradient ones column is not counted)."""
    G, T, B, H, D = GATES[w.mode], w.T, w.B, w.hidden, w.dirs
    f = {"gemm_input": 0.0, "gemm_dx": 0.0, "gemm_dw": 0.0, "recurrent_fwd": 0.0, "recurrent_bwd": 0.0}
    for l in range(w.layers):
        I_l = w.input_size if l == 0 else D * H
        f["gemm_input"] += 2.0 * T * B * D * G * H * I_l
        f["gemm_dx"] += 2.0 * T * B * D * G * H * I_l
        f["gemm_dw"] += 2.0 * T * B * D * G * H * (I_l + H)
        f["recurrent_fwd"] += 2.0 * T * B * D * G * H * H
        f["recurrent_bwd"] += 2.0 * T * B * D * G * H * H
    return f


def timed_region(torch, fn, steps, warmup):
    """W untimed steps, then exactly K steps bracketed by synchronisations:
    (ms per step from events around the K steps, wall seconds)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps, time.perf_counter() - t0


def kernel_breakdown(run, torch, R, steps):
    """Per-kernel launch times from the HIP events the library records on the
    caller's stream around each launch (a separate pass: the events are off
    while the headline is timed)."""
    R.rnn_set_profiling(run.h, True)
    for _ in range(steps):
        run.train_step()
    torch.cuda.synchronize()
    kern = {}
    for k, name in enumerate(R.KERNEL_NAMES):
        n, ms = R.rnn_profile_read(run.h, k)
        if n:
            kern[name] = {"launches": n, "avg_us": round(1000 * ms / n, 3), "total_ms": round(ms, 3)}
    R.rnn_set_profiling(run.h, False)
    assert R.rnn_device_status(run.h, run.ws) == 0
    return kern


def exchange_floor(run, w, R, reps):
    """The training forward sweep's launch with only its exchange (flag
    waits, ring stores, flags), per step: the recurrence's latency floor."""
    try:
        R.rnn_set_profiling(run.h, True)
        for _ in range(reps):
            R.rnn_exchange_floor(run.h, w.T, w.B, run.ws, training=True)
        n_p, ms_p = R.rnn_profile_read(run.h, R.KERNEL_NAMES.index("exchange_probe"))
        R.rnn_set_profiling(run.h, False)
        assert R.rnn_device_status(run.h, run.ws) == 0
        steps_per_sweep = w.T + (w.layers - 1 if w.dirs == 1 and w.layers > 1 else 0)
        return 1000.0 * ms_p / n_p / steps_per_sweep
    except R.RNNError:   # the sweep could not run persistently
        R.rnn_set_profiling(run.h, False)
        return None


def kernel_rooflines(w, kern, steps, floor_us):
    """One entry per kernel kind: the time-parallel products against the
    dense MFMA peak of their operand type; the recurrent sweeps, bound by
    their per-step latency, against the measured exchange floor (their
    fraction of the MFMA peak is given too)."""
    peak = PEAK_TFLOPS[w.wtype]
    fl = kernel_flops(w)
    sweeps_per_step = {"recurrent_fwd": 1 if (w.dirs == 1 and w.layers > 1) else w.layers,
                       "recurrent_bwd": w.layers}
    out = {}
    for name, f in fl.items():
        k = kern.get(name)
        if not k:
            continue
        t_step = k["total_ms"] / steps * 1e-3    # seconds of this kernel kind per training step
        achieved = f / t_step / 1e12
        e = {"achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
             "frac_mfma_peak": round(achieved / peak, 5), "avg_launch_us": k["avg_us"],
             "launches_per_step": round(k["launches"] / steps, 2), "flops_per_step": f}
        if name.startswith("recurrent"):
            steps_per_sweep = w.T + (w.layers - 1 if name == "recurrent_fwd" and w.dirs == 1 and w.layers > 1 else 0)
            us_step = k["total_ms"] / steps * 1000.0 / sweeps_per_step[name] / steps_per_sweep
            e.update(bound="latency", us_per_recurrent_step=round(us_step, 3))
            if floor_us:
                e.update(exchange_floor_us_per_step=round(floor_us, 3),
                         frac_of_latency_floor=round(floor_us / us_step, 4))
        else:
            e["bound"] = "mfma"
        out[name] = e
    return out


def measure(w, torch, R, synth, steps, warmup, dropout=0.0, detail=True):
    run = Runner(w, torch, R, synth, dropout=dropout)
    F_train = 3 * flops(w.mode, w.T, w.B, w.input_size, w.hidden, w.layers, w.dirs)
    fwd_ms, _ = run.timed(run.fwd, max(5, steps // 2), warmup)
    T_ms, wall = timed_region(torch, run.train_step, steps, warmup)
    assert R.rnn_device_status(run.h, run.ws) == 0
    value = F_train / (T_ms * 1e-3) / 1e9
    r = {"value": round(value, 3), "ms_per_step": round(T_ms, 4), "wall_s": round(wall, 4),
         "fwd_ms": round(float(np.median(fwd_ms)), 4),
         "pct_mfma_peak": round(100.0 * value / (PEAK_TFLOPS[w.wtype] * 1000.0), 4)}
    if not detail:
        return run, r
    step_ms, _ = run.timed(run.train_step, steps, 0)   # per-step spread (events per step)
    r["train_step_ms_p10_p50_p90"] = [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)]
    r["kernels"] = kernel_breakdown(run, torch, R, steps)
    r["plan"] = R.rnn_plan_info(run.h, w.T, w.B, True)
    return run, r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lstm_ds2_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fp32", action="store_true")
    ap.add_argument("--no-small-batch", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the stacked / GRU workloads reported next to the headline")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time the vendor BLAS on the same GEMM shapes (context only)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="inter-layer dropout probability of the training steps")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build "
              "(the operator has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import layer_rnn_forward_amd as R
    from layer_rnn_forward_amd import synth

    w = synth.WORKLOADS[args.workload]
    run, m = measure(w, torch, R, synth, args.steps, args.warmup, dropout=args.dropout)
    kern = m["kernels"]
    floor = exchange_floor(run, w, R, max(3, args.steps // 4))
    peak = PEAK_TFLOPS[w.wtype]
    roofs = kernel_rooflines(w, kern, args.steps, floor)

    # the dominant kernel: the kind with the largest total time
    dname, dk = max(kern.items(), key=lambda kv: kv[1]["total_ms"])
    fl = kernel_flops(w)
    if dname in fl:
        per_launch = fl[dname] * args.steps / dk["launches"]
        achieved = per_launch / (dk["avg_us"] * 1e-6) / 1e12
        roof = {"kernel": dname, "bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 5),
                "traffic": measured_traffic(dname) if w.name == "lstm_ds2_bf16" else None,
                "avg_launch_us": dk["avg_us"], "algorithmic_flops_per_launch": per_launch}
        if dname.startswith("recurrent"):
            # a step-serial recurrence: its time is set by the per-step latency
            # (exchange round trip, fragment loads, cell math), not by MFMA or
            # HBM throughput; the MFMA fraction above is the contract's figure
            roof["limiter"] = "per-step latency of the recurrence (exchange-bound)"
            roof["us_per_recurrent_step"] = roofs[dname]["us_per_recurrent_step"]
            roof["exchange_floor_us_per_step"] = round(floor, 3) if floor else None
    else:
        roof = {"kernel": dname, "bound": "mfma", "achieved": None, "peak": peak, "unit": "TFLOP/s",
                "frac": None, "traffic": None, "avg_launch_us": dk["avg_us"]}

    out = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.wtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian inputs, uniform weights; no data set)",
        "config": {"workload": w.name, "mode": w.mode, "layers": w.layers, "dirs": w.dirs,
                   "T": w.T, "B": w.B, "input": w.input_size, "hidden": w.hidden,
                   "weights": w.wtype, "state_accum": "f32", "dropout": args.dropout},
        "fwd_ms": m["fwd_ms"],
        "pct_mfma_peak": m["pct_mfma_peak"],
        "timed_wall_s": m["wall_s"],
        "train_step_ms_p10_p50_p90": m["train_step_ms_p10_p50_p90"],
        "kernels": kern,
        "roofline": roof,
        "kernel_rooflines": roofs,
        "plan": m["plan"],
        "source_sha16": source_hash(),
    }
    if floor:
        fwd_step = roofs["recurrent_fwd"]["us_per_recurrent_step"]
        out["exchange_floor"] = {"floor_us_per_step": round(floor, 3), "recurrent_fwd_us_per_step": fwd_step,
                                 "floor_fraction_of_step": round(floor / fwd_step, 4)}
    # measured denominators next to the published peaks
    probes = {k: mfma_peak(torch, R, k) for k in R.MFMA_PROBES}
    meas = {"bf16": max(probes["bf16_16x16x32"], probes["bf16_32x32x16"]), "f32": probes["f32_16x16x4"]}
    out["mfma_peak_measured"] = {**{f"{k}_TFLOPs": round(v, 1) for k, v in probes.items()},
                                 "published_bf16_TFLOPs": PEAK_TFLOPS["bf16"],
                                 "published_f32_TFLOPs": PEAK_TFLOPS["f32"]}
    out["pct_measured_mfma_peak"] = round(100.0 * m["value"] / (meas[w.wtype] * 1000.0), 4)
    if args.dropout == 0.0:   # (a captured step would replay one dropout seed)
        try:
            g_ms = run.graph_timed(args.steps, args.warmup)
            assert R.rnn_device_status(run.h, run.ws) == 0
            F_train = 3 * flops(w.mode, w.T, w.B, w.input_size, w.hidden, w.layers, w.dirs)
            out["graph_replay"] = {"ms_per_step": round(g_ms, 4),
                                   "value": round(F_train / (g_ms * 1e-3) / 1e9, 3), "unit": "GFLOP/s",
                                   "note": "the same training step captured once into a HIP graph and replayed"}
        except (RuntimeError, R.RNNError) as e:   # capture unavailable: report, keep the eager line
            torch.cuda.synchronize()
            out["graph_replay"] = {"error": str(e)}
    if "dropout" in kern:
        # HBM-bound pass: reads and writes one fp32 per element of a layer input
        n_el = w.T * w.B * w.dirs * w.hidden
        gbs = 8.0 * n_el / (kern["dropout"]["avg_us"] * 1e-6) / 1e9
        out["dropout_pass"] = {"avg_us": kern["dropout"]["avg_us"], "bytes_per_launch": 8 * n_el,
                               "achieved_GBs": round(gbs, 1), "frac_hbm": round(gbs / HBM_GBS, 4)}
    del run
    if not args.no_fp32 and w.wtype == "bf16" and args.dropout == 0.0:
        w32 = synth.WORKLOADS.get(args.workload.replace("bf16", "f32"))
        if w32 is not None:
            r32, m32 = measure(w32, torch, R, synth, args.steps, args.warmup, detail=False)
            del r32
            out["fp32_weights"] = {"value": m32["value"], "unit": "GFLOP/s", "ms_per_step": m32["ms_per_step"],
                                   "fwd_ms": m32["fwd_ms"], "pct_mfma_peak": m32["pct_mfma_peak"],
                                   "pct_measured_mfma_peak": round(100.0 * m32["value"] / (meas["f32"] * 1000), 4)}
    if not args.no_secondary and args.workload == "lstm_ds2_bf16" and args.dropout == 0.0:
        # the other workloads: GRU, 5-layer bidirectional stacks, the
        # unidirectional 5-layer stack (layer wavefront); same step and timing
        sec = {}
        for name in SECONDARY:
            ws_ = synth.WORKLOADS[name]
            r2, m2 = measure(ws_, torch, R, synth, max(5, args.steps // 2), args.warmup, detail=False)
            k2 = kernel_breakdown(r2, torch, R, 3)
            del r2
            sec[name] = {"mode": ws_.mode, "layers": ws_.layers, "dirs": ws_.dirs, "weights": ws_.wtype,
                         "value": m2["value"], "unit": "GFLOP/s", "ms_per_step": m2["ms_per_step"],
                         "fwd_ms": m2["fwd_ms"], "pct_mfma_peak": m2["pct_mfma_peak"],
                         "pct_measured_mfma_peak": round(100.0 * m2["value"] / (meas[ws_.wtype] * 1000.0), 4),
                         "kernel_ms_per_step": {k: round(v["total_ms"] / 3, 4) for k, v in k2.items()}}
        out["workloads"] = sec
    if not args.no_small_batch and w.layers == 1:
        # serving-size batches: forward-inference latency of the same layer,
        # and of the vanilla tanh RNN of the same size (whose small batches
        # get XCD-local recurrence groups)
        import dataclasses

        def serving(wb):
            sb = {}
            for Bs in (1, 2, 4):
                rs = Runner(dataclasses.replace(wb, B=Bs), torch, R, synth)
                f_ms, _ = rs.timed(rs.fwd, max(5, args.steps // 2), args.warmup)
                med = float(np.median(f_ms))
                sb[str(Bs)] = {"fwd_ms": round(med, 4), "us_per_step": round(1000.0 * med / wb.T, 3),
                               "plan": R.rnn_plan_info(rs.h, wb.T, Bs, False)["fwd"]}
                del rs
            return sb

        out["small_batch_fwd"] = serving(w)
        if w.mode != "rnn_tanh":
            out["small_batch_fwd_tanh"] = serving(dataclasses.replace(w, mode="rnn_tanh", name=w.name + "_tanh"))
    if args.blas_reference and w.wtype == "bf16":
        out["vendor_gemm_reference"] = blas_reference(torch, w)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, synth, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
