#!/usr/bin/env python3
"""Throughput of the stacked-LSTM forward pass on one MI355X.

One step = one lstm_fwd call: the whole forward pass (every layer, every
timestep) over one batch of the seeded synthetic workload, inputs resident in
HBM.  Prints one JSON line:

  value        TFLOP/s of the whole step, FLOPs = sum_l 2*4H*(I_l+H)*B*T,
               over the mean step time (K steps between two HIP events)
  ms_per_sequence  the median time of one call (one forward over B sequences)
  roofline     the dominant kernel: its algorithmic work per launch (FLOPs,
               or the bytes of its binding memory level) over its mean launch
               time (HIP events the library records on its own stream), against
               the MI355X published peak of the binding resource (dense MFMA of
               the dtype, HBM, or LDS for weights re-read from LDS every step)
  phases       the input projections and the recurrence of one step, each
               against its own roofline and the MFMA peak
  measured_peaks  MFMA / HBM / LDS rates measured on the same box
  cpu_baseline the fp64 oracle timed on the host cores (a baseline only)

Default workload: 4-layer LSTM, I = H = 4096, B = 32, T = 50, bf16 (fp32
accumulation and cell state), the largest of the five.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}  # MI355X dense MFMA, published
WORKLOAD_TEXT = {
    "c1": "1-layer LSTM I=H=128 B=8 T=16 fp32",
    "c2": "4-layer LSTM I=H=512 B=64 T=100 fp32",
    "c3": "8-layer LSTM I=H=256 B=64 T=200 bf16 (fp32 accumulate and cell state)",
    "c4": "4-layer LSTM I=H=4096 B=32 T=50 bf16 (fp32 accumulate and cell state)",
    "c5": "1-layer LSTM I=H=1536 B=4 T=2048 bf16 (fp32 accumulate and cell state)",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def launch_layer(plan: dict, kind: int, launch_index: int) -> int:
    """Layer of a layerwise run's launch `launch_index` (input GEMM, recurrence, ... per layer)."""
    return 0 if plan["regime"] == "wavefront" else launch_index // 2


def kernel_model(cfg, kind: int, plan: dict, launch_index: int) -> dict:
    """Algorithmic work of one launch: FLOPs (2 per multiply-add; bias and gate
    math excluded), the HBM bytes the method must move, and the LDS bytes its
    weight reads take when the weights stay in LDS for the whole sequence.

    G*H weight rows per matrix: G = 4 (LSTM), 3 (GRU), 1 (simple RNN); s bytes
    per element.  Per kind:
      input GEMM of layer l   flops 2*G*H*I_l*T*B; HBM W_l + U + G (fp32 out)
      layerwise recurrence    flops 2*G*H*H*B*T; HBM R_l once when it stays on
                              chip (T times when streamed) + G read + h written;
                              LDS the part of R_l held in LDS, read every step
      wavefront recurrence    every layer's R h plus the fused W u products;
                              HBM weights once + x + y; LDS every layer's
                              [W_l | R_l] read every step
    """
    H, B, T, L, I, G = cfg.H, cfg.B, cfg.T, cfg.L, cfg.I, cfg.gates
    s = 2 if cfg.dtype == "bf16" else 4
    rows = G * H
    g_bytes = T * 4 * H * B * 4  # hoisted pre-activations, fp32, 16-row tiles of 4 rows per unit
    if cfg.cell in ("rnn_tanh", "rnn_relu"):
        g_bytes = T * H * B * 4
    if kind == 1:
        il = I if launch_layer(plan, kind, launch_index) == 0 else H
        return {"flops": 2.0 * rows * il * B * T, "hbm": rows * il * s + T * B * il * s + g_bytes, "lds": 0.0}
    if kind != 2:  # clearing the step counters
        return {"flops": 0.0, "hbm": 0.0, "lds": 0.0}
    if plan["regime"] == "wavefront":
        fused_in = (I + (L - 1) * H) if plan["input_gemms"] == 0 else (L - 1) * H
        w_bytes = (L * rows * H + rows * fused_in) * s
        return {"flops": 2.0 * rows * H * B * T * L + 2.0 * rows * fused_in * B * T,
                "hbm": w_bytes + T * B * I * s + T * B * H * s,
                "lds": float(T) * w_bytes if plan["weights_on_chip"] else 0.0}
    r_bytes = rows * H * s
    nrb = plan.get("weight_blocks_in_registers", 0)
    if plan["weights_streamed"]:
        lds, hbm_r = 0.0, T * r_bytes
    elif nrb:  # register-resident: a quarter of each wave's blocks in LDS (16 of 64)
        lds, hbm_r = float(T) * r_bytes * (1.0 - nrb / 64.0), r_bytes
    else:
        lds, hbm_r = float(T) * r_bytes, r_bytes
    return {"flops": 2.0 * rows * H * B * T, "hbm": hbm_r + g_bytes + T * B * H * s, "lds": lds}


def kernel_name(kind: int, plan: dict) -> str:
    if kind == 1:
        return "lstm_input_gemm"
    if kind == 2:
        return "lstm_rec_res_kernel" if plan.get("weight_blocks_in_registers", 0) else "lstm_rec_kernel"
    return "lstm_clear"


def roofline_of(model: dict, ms: float, peaks: dict, dtype: str) -> dict:
    """The binding roof of one launch (the resource whose algorithmic time is
    longest at its peak) and the achieved rate on it."""
    t = {"mfma": model["flops"] / (peaks["mfma"][dtype] * 1e12),
         "hbm": model["hbm"] / (peaks["hbm"] * 1e9),
         "lds": model["lds"] / (peaks["lds"] * 1e9)}
    bound = max(t, key=t.get)
    if bound == "mfma":
        ach, peak, unit, per = model["flops"] / (ms * 1e-3) / 1e12, peaks["mfma"][dtype], "TFLOP/s", model["flops"]
    else:
        ach, peak, unit, per = model[bound] / (ms * 1e-3) / 1e9, peaks[bound], "GB/s", model[bound]
    return {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak, "per_launch": per,
            "floor_ms": t[bound] * 1e3}


# Sources the forward's kernels are not built from (the backward pass, the
# peak microbenchmarks, the allocation-free entry point's wrapper).
DIGEST_EXCLUDED = ("lstm_bwd.hip", "lstm_bwd_res.h", "lstm_bwd_res_inst.hip", "lstm_peaks.hip",
                   "lstm_fwd_noalloc.hip")


def kernel_source_digest() -> str:
    """sha256 over the forward's sources (kernels, planner, launch code): HBM
    counter figures taken for other sources no longer describe the kernel."""
    import hashlib
    csrc = os.path.join(ROOT, "stacked_lstm_forward_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".h", ".hip", ".cpp")) and fn not in DIGEST_EXCLUDED:
            h.update(fn.encode())
            h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summaries in profiles/ (a line 'bench-traffic: {json}'), or None when there
    is none for the current sources."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    digest = kernel_source_digest()
    for fn in sorted(os.listdir(pdir)):
        if not fn.endswith((".md", ".txt")):
            continue
        for line in open(os.path.join(pdir, fn)):
            if not line.startswith("bench-traffic:"):
                continue
            try:
                rec = json.loads(line.split(":", 1)[1])
            except ValueError:
                continue
            if rec.get("workload") == workload and rec.get("kernel") == kernel and rec.get("source_sha256") == digest:
                return int(rec["fetch_bytes"] + rec["write_bytes"])
    return None


def blas_info():
    """(threads the BLAS pool runs, vendor) of the NumPy the oracle uses."""
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        if pools:
            return max(p.get("num_threads", 1) for p in pools), pools[0].get("internal_api", "unknown")
    except Exception:  # pragma: no cover
        pass
    return os.cpu_count() or 1, "unknown"


def cpu_baseline(inp, cfg, min_seconds: float) -> dict:
    """The fp64 oracle on the host cores, on a bounded sample of the workload:
    every layer and every sequence, the first T_s of the T steps (the work per
    step is the same at every step, so FLOPs scale with T_s).  T_s is sized
    from a one-step probe so that the timed run takes about `min_seconds`."""
    import dataclasses
    import lstm_inputs as li
    from oracle.lstm_oracle import forward_inputs
    threads, vendor = blas_info()

    def sub(ts):
        c = li.Config(f"{cfg.name}-T{ts}", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, ts, cfg.dtype, cfg.cell)
        return dataclasses.replace(inp, cfg=c, x=inp.x[:ts]), c

    probe, _ = sub(1)
    t0 = time.perf_counter()
    forward_inputs(probe)
    per_step = max(time.perf_counter() - t0, 1e-6)
    ts = max(1, min(cfg.T, int(min_seconds / per_step)))
    sample, scfg = sub(ts)
    reps, t0 = 0, time.perf_counter()
    while True:
        forward_inputs(sample)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 50:
            break
    what = "the whole workload" if ts == cfg.T else f"all {cfg.L} layers and {cfg.B} sequences, the first {ts} of {cfg.T} steps"
    return {"value": scfg.flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} ({scfg.flops / 1e9:.1f} GFLOP) run {reps}x by the fp64 NumPy oracle in {el:.1f} s",
            "blas": vendor, "host_cpus": len(os.sched_getaffinity(0)), "precision": "fp64",
            "ms_per_forward_extrapolated": round(el / reps * cfg.T / ts * 1e3, 1)}


def train_bench(args, cfg, workload, inp) -> int:
    """One training step = lstm_fwd_train (the forward that keeps gates, cell and
    hidden states) + lstm_bwd (backpropagation through time, weight gradients as
    single products over all T*B columns), timed with events on the stream the
    library enqueues on.  FLOPs: the forward's, plus twice that for the backward
    (the recurrent chain dP R, and dW, dR and the input gradient dP W)."""
    import numpy as np
    import torch
    from stacked_lstm_forward_amd import runner
    if cfg.cell != "lstm":
        print("--train covers the LSTM cell", file=sys.stderr)
        return 2
    rng = np.random.default_rng(1234)
    dy = rng.standard_normal((cfg.T, cfg.B, cfg.H)).astype(np.float32)
    dhT = rng.standard_normal((cfg.L, cfg.B, cfg.H)).astype(np.float32)
    dcT = rng.standard_normal((cfg.L, cfg.B, cfg.H)).astype(np.float32)
    tp = runner.prepare_train(inp, dy, dhT, dcT, "cuda:0")
    stream = torch.cuda.current_stream()
    plain = bool(args.plain_launch)
    for _ in range(args.warmup):
        tp.forward(stream, plain)
        tp.backward(stream, plain)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for k in range(args.steps):
        ev[k][0].record(stream)
        tp.forward(stream, plain)
        ev[k][1].record(stream)
        tp.backward(stream, plain)
        ev[k][2].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    st = sl_last_error(tp.fwd)
    if not st:
        import stacked_lstm_forward_amd as sl
        b = sl.lstm_bwd_last_error(tp.bws)
        st = "" if b == sl.LSTM_OK else sl.lstm_status_string(b)
    if st:
        print(f"timed training run failed: {st}", file=sys.stderr)
        return 1
    ms_step = t0.elapsed_time(t1) / args.steps
    fwd = median([e[0].elapsed_time(e[1]) for e in ev])
    bwd = median([e[1].elapsed_time(e[2]) for e in ev])
    g = tp.grads_f64()
    if not all(np.all(np.isfinite(v)) for v in (g["dx"], g["dh0"], g["dc0"], *g["dW"], *g["dR"], *g["db"])):
        print("non-finite gradients", file=sys.stderr)
        return 1
    dt = "f32" if cfg.dtype == "f32" else "bf16"
    peak = SPEC_PEAKS["mfma"][dt]
    flops = 3 * cfg.flops
    value = flops / (ms_step * 1e-3) / 1e12
    bwd_tf = 2 * cfg.flops / (bwd * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 backward oracle on the host (cpu_baseline)")
        cpu = cpu_baseline_train(inp, cfg, dy, dhT, dcT, args.cpu_seconds)
    out = {
        "metric": "stacked-LSTM training step (forward keeping state + backward) TFLOPS",
        "value": round(value, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dt, "data": "synthetic (seeded; dy, dhT, dcT ~ N(0,1))",
        "config": {"workload": workload, "cell": cfg.cell, "L": cfg.L, "I": cfg.I, "H": cfg.H, "B": cfg.B,
                   "T": cfg.T, "gflop_per_step": round(flops / 1e9, 3)},
        "roofline": {"bound": "mfma", "achieved": round(bwd_tf, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(bwd_tf / peak, 4), "traffic": None, "kernel": "lstm_bwd (all its kernels)",
                     "ms_per_launch": round(bwd, 5), "algorithmic_per_launch": 2 * cfg.flops},
        "phases": {"forward_train": {"ms_median": round(fwd, 5),
                                     "tflops": round(cfg.flops / (fwd * 1e-3) / 1e12, 2)},
                   "backward": {"ms_median": round(bwd, 5), "tflops": round(bwd_tf, 2),
                                "frac_of_mfma_peak": round(bwd_tf / peak, 4)}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def sl_last_error(prob) -> str:
    import stacked_lstm_forward_amd as sl
    st = sl.lstm_fwd_last_error(prob.ws, None)
    return "" if st == sl.LSTM_OK else sl.lstm_status_string(st)


def cpu_baseline_train(inp, cfg, dy, dhT, dcT, min_seconds: float) -> dict:
    """The fp64 backward oracle (its forward included) on a bounded sample:
    every layer and sequence, the first T_s steps."""
    import dataclasses
    import lstm_inputs as li
    from oracle.lstm_oracle_bwd import lstm_backward_inputs
    threads, vendor = blas_info()

    def sub(ts):
        c = li.Config(f"{cfg.name}-T{ts}", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, ts, cfg.dtype, cfg.cell)
        return dataclasses.replace(inp, cfg=c, x=inp.x[:ts]), c

    probe, _ = sub(1)
    t0 = time.perf_counter()
    lstm_backward_inputs(probe, dy[:1], dhT, dcT)
    per_step = max(time.perf_counter() - t0, 1e-6)
    ts = max(1, min(cfg.T, int(min_seconds / per_step)))
    sample, scfg = sub(ts)
    reps, t0 = 0, time.perf_counter()
    while True:
        lstm_backward_inputs(sample, dy[:ts], dhT, dcT)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 50:
            break
    return {"value": 3 * scfg.flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"all {cfg.L} layers and {cfg.B} sequences, the first {ts} of {cfg.T} steps, forward and "
                      f"backward ({3 * scfg.flops / 1e9:.1f} GFLOP) run {reps}x by the fp64 NumPy oracle in {el:.1f} s",
            "blas": vendor, "host_cpus": len(os.sched_getaffinity(0)), "precision": "fp64"}


# The pages' own figures, on other hardware: context, never a target.
PAGES_CONTEXT = {
    "naive_rnn_tflops_m40": 0.4, "m40_peak_tflops": 5.8, "after_gate_grouping_tflops_m40": 0.8,
    "gpu_vs_mkl_cpu_speedup": "2-11x (a separate large-scale RNN work; GPU not stated)",
    "sources": ["Optimizing Performance of Recurrent Neural Networks on GPUs (key results)",
                "Large Scale Recurrent Neural Network on GPU (abstract)"],
}

# MI355X published peaks (dense MFMA, HBM3E) and the LDS read rate of CDNA4
# (256 CUs x 256 bytes per clock x 2.4 GHz; the microbenchmark measures about
# 132 TB/s, above what 128 bytes per clock could give).
SPEC_PEAKS = {"mfma": {"f32": 157.3, "bf16": 2516.6}, "hbm": 8000.0, "lds": 157286.4}


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--cell", default="lstm", choices=["lstm", "gru", "rnn_tanh", "rnn_relu"],
                    help="recurrent cell at the workload's shapes (the headline metric is the LSTM)")
    ap.add_argument("--regime", type=int, default=0, help="0 auto, 1 layerwise, 2 wavefront")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (calibrates HBM traffic counters)")
    ap.add_argument("--plain-launch", action="store_true",
                    help="ordinary (not cooperative) launch of the persistent kernel, for profilers")
    ap.add_argument("--train", action="store_true",
                    help="time a training step (lstm_fwd_train + lstm_bwd) instead of the forward")
    ap.add_argument("--source-digest", action="store_true",
                    help="print the digest of the library sources that counter summaries are keyed on")
    args = ap.parse_args()

    if args.source_digest:
        print(kernel_source_digest())
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the forward pass runs on a single MI355X and the library "
              "has no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import lstm_inputs as li
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 1
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}), flush=True)
        return 0
    sl.load_library()
    cfg = li.CONFIGS[args.config]
    workload = WORKLOAD_TEXT[cfg.name]
    if args.cell != "lstm":
        cfg = li.with_cell(cfg, args.cell)
        workload = workload.replace("LSTM", args.cell.upper().replace("_", "-"))
    log(f"workload {cfg.name}: {workload}; generating inputs")
    inp = li.make_inputs(cfg)
    if args.train:
        return train_bench(args, cfg, workload, inp)
    prob = runner.prepare(inp, "cuda:0")
    plan = sl.lstm_fwd_plan(prob.desc, args.regime).as_dict()
    log(f"plan {plan}")

    stream = torch.cuda.current_stream()
    maxl = 16
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * maxl)] for _ in range(args.steps)]
    for row in evs:  # torch creates the HIP event on first record
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    kinds = [(ctypes.c_int32 * maxl)() for _ in range(args.steps)]
    nls = [ctypes.c_int32(0) for _ in range(args.steps)]
    opts_list = []
    keep = []
    for k in range(args.steps):
        st_arr = (ctypes.c_void_p * maxl)(*[e.cuda_event for e in evs[k][:maxl]])
        sp_arr = (ctypes.c_void_p * maxl)(*[e.cuda_event for e in evs[k][maxl:]])
        keep += [st_arr, sp_arr]
        o = sl.LstmOpts()
        o.force_regime = args.regime
        o.plain_launch = 1 if args.plain_launch else 0
        o.max_launches = maxl
        o.ev_start = ctypes.cast(st_arr, ctypes.POINTER(ctypes.c_void_p))
        o.ev_stop = ctypes.cast(sp_arr, ctypes.POINTER(ctypes.c_void_p))
        o.launch_kind = kinds[k]
        o.num_launches = ctypes.pointer(nls[k])
        opts_list.append(o)
    plain = sl.LstmOpts()
    plain.force_regime = args.regime
    plain.plain_launch = 1 if args.plain_launch else 0

    for _ in range(args.warmup):
        prob.run(stream, plain)
    torch.cuda.synchronize()
    st = sl.lstm_fwd_last_error(prob.ws, stream)
    if st != sl.LSTM_OK:
        print(f"warm-up failed: {sl.lstm_status_string(st)}", file=sys.stderr)
        return 1
    log(f"warm-up done ({args.warmup} steps); timing {args.steps} steps")

    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e in step_ev:
        e.record(stream)
    torch.cuda.synchronize()
    t_start.record(stream)
    step_ev[0].record(stream)
    for k in range(args.steps):
        prob.run(stream, opts_list[k])
        step_ev[k + 1].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    st = sl.lstm_fwd_last_error(prob.ws, stream)
    if st != sl.LSTM_OK:
        print(f"timed run failed: {sl.lstm_status_string(st)}", file=sys.stderr)
        return 1
    total_ms = t_start.elapsed_time(t_stop)
    ms_step = total_ms / args.steps
    per_step = sorted(step_ev[k].elapsed_time(step_ev[k + 1]) for k in range(args.steps))
    ms_median = median(per_step)

    # per-launch durations from the library's launch events (recorded on the
    # stream the kernels run on), grouped by kernel and by phase
    per_kind: dict = {}
    model_kind: dict = {}
    phase_ms = {1: [], 2: [], 3: []}
    for k in range(args.steps):
        n = nls[k].value
        acc = {1: 0.0, 2: 0.0, 3: 0.0}
        for j in range(n):
            kind = kinds[k][j]
            d = evs[k][j].elapsed_time(evs[k][maxl + j])
            per_kind.setdefault(kind, []).append(d)
            model_kind.setdefault(kind, []).append(kernel_model(cfg, kind, plan, j))
            acc[kind] = acc.get(kind, 0.0) + d
        for kind in phase_ms:
            phase_ms[kind].append(acc.get(kind, 0.0))
    value = cfg.flops / (ms_step * 1e-3) / 1e12
    y, hT, cT = prob.outputs_f32()
    import numpy as np
    if not (np.all(np.isfinite(y)) and np.all(np.isfinite(hT)) and (cT is None or np.all(np.isfinite(cT)))):
        print("non-finite outputs", file=sys.stderr)
        return 1

    # measured peaks of this machine (microbenchmarks), beside the published ones
    measured = None
    if not args.no_peaks:
        try:
            from stacked_lstm_forward_amd import peaks as pk
            log("measuring MFMA, HBM and LDS peaks (microbenchmarks)")
            measured = pk.measure_peaks()
        except Exception as e:  # the forward's figures stand without them
            log(f"peak microbenchmarks unavailable: {e}")
    dt = "f32" if cfg.dtype == "f32" else "bf16"

    def mean(v):
        return sum(v) / len(v)

    dom = max(per_kind, key=lambda kk: sum(per_kind[kk]))
    dom_ms = mean(per_kind[dom])
    dom_model = {key: mean([m[key] for m in model_kind[dom]]) for key in ("flops", "hbm", "lds")}
    rl = roofline_of(dom_model, dom_ms, SPEC_PEAKS, dt)
    roof = {"bound": rl["bound"], "achieved": round(rl["achieved"], 3), "peak": rl["peak"], "unit": rl["unit"],
            "frac": round(rl["frac"], 4),
            "traffic": measured_traffic(cfg.name, kernel_name(dom, plan)),
            "kernel": kernel_name(dom, plan), "ms_per_launch": round(dom_ms, 5),
            "algorithmic_per_launch": rl["per_launch"], "floor_ms_per_launch": round(rl["floor_ms"], 5)}
    if measured:
        mpk = {"mfma": measured["mfma_tflops"], "hbm": measured["hbm_gbs"], "lds": measured["lds_gbs"]}
        mpk_dt = {"mfma": {dt: mpk["mfma"][dt]}, "hbm": mpk["hbm"], "lds": mpk["lds"]}
        rlm = roofline_of(dom_model, dom_ms, mpk_dt, dt)
        roof["peak_measured"] = round(rlm["peak"], 1)
        roof["frac_of_measured_peak"] = round(rl["achieved"] / (mpk["mfma"][dt] if rl["bound"] == "mfma"
                                                                else mpk[rl["bound"]]), 4)
    log(f"{ms_step:.4f} ms/step, {value:.2f} TFLOP/s; dominant kernel {roof['kernel']}: {dom_ms:.4f} ms/launch, "
        f"{rl['bound']} bound, frac {rl['frac']:.4f}")

    # phases of the forward: every launch of a kind per step (median over steps)
    phases = {}
    for kind, name in ((1, "input_projection"), (2, "recurrence")):
        if not per_kind.get(kind):
            continue
        ms = median(phase_ms[kind])
        fl = sum(m["flops"] for m in model_kind[kind]) / args.steps
        ent = {"kernel": kernel_name(kind, plan), "launches_per_step": len(per_kind[kind]) // args.steps,
               "ms_per_step": round(ms, 5), "ms_per_launch": round(mean(per_kind[kind]), 5),
               "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
               "frac_of_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / SPEC_PEAKS["mfma"][dt], 4)}
        lm = {key: mean([m[key] for m in model_kind[kind]]) for key in ("flops", "hbm", "lds")}
        rk = roofline_of(lm, mean(per_kind[kind]), SPEC_PEAKS, dt)
        ent["bound"] = rk["bound"]
        ent["frac_of_roofline"] = round(rk["frac"], 4)
        if measured:
            ent["frac_of_measured_mfma_peak"] = round(ent["tflops"] / measured["mfma_tflops"][dt], 4)
        phases[name] = ent

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host (cpu_baseline)")
        cpu = cpu_baseline(inp, cfg, args.cpu_seconds)
        log(f"cpu_baseline {cpu}")

    out = {
        "metric": "stacked-LSTM fwd TFLOPS (% of MI355X roofline) and ms/sequence",
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "ms_per_step_min": round(per_step[0], 5),
        # one call runs the whole forward over the batch of B sequences: its
        # median time, and that time divided by B
        "ms_per_sequence": round(ms_median, 5),
        "ms_per_sequence_div_B": round(ms_median / cfg.B, 6),
        "tflops_at_median": round(cfg.flops / (ms_median * 1e-3) / 1e12, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded: W,R,b ~ U(-1/sqrt(H),1/sqrt(H)), x ~ N(0,1), h0=c0=0)",
        "config": {"workload": workload, "cell": cfg.cell, "L": cfg.L, "I": cfg.I, "H": cfg.H, "B": cfg.B,
                   "T": cfg.T, "regime": plan["regime"], "gflop_per_step": round(cfg.flops / 1e9, 3)},
        "roofline": roof,
        "whole_forward_frac_of_mfma_peak": round(value / SPEC_PEAKS["mfma"][dt], 4),
        "phases": phases,
        "kernels_ms_per_launch": {kernel_name(kk, plan): round(mean(v), 5) for kk, v in per_kind.items()},
        "measured_peaks": measured,
        "cpu_baseline": cpu,
        "pages_context": PAGES_CONTEXT,
    }
    if measured:
        out["whole_forward_frac_of_measured_mfma_peak"] = round(value / measured["mfma_tflops"][dt], 4)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
