#!/usr/bin/env python3
"""Throughput of the stacked-LSTM forward pass on one MI355X.

One step = one lstm_fwd call: the whole forward pass (every layer, every
timestep) over one batch of the seeded synthetic workload, inputs resident in
HBM.  Prints one JSON line:

  value        TFLOP/s of the whole step, FLOPs = sum_l 2*4H*(I_l+H)*B*T
  ms_per_step  mean wall time of one step (HIP events around K steps)
  roofline     the dominant kernel: algorithmic FLOPs per launch / its mean
               launch time (HIP events the library records on its stream),
               against the MI355X dense MFMA peak of the workload's dtype
  cpu_baseline the fp64 oracle timed on the host cores (a baseline only)

Default workload: 4-layer LSTM, I = H = 512, B = 64, T = 100, fp32.
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


def kernel_flops(cfg, kind: int, plan: dict, launch_index: int) -> float:
    """Algorithmic FLOPs of one launch (2 per multiply-add; bias and gate math excluded).
    G*H weight rows per matrix: G = 4 (LSTM), 3 (GRU), 1 (simple RNN)."""
    H, B, T, L, I, G = cfg.H, cfg.B, cfg.T, cfg.L, cfg.I, cfg.gates
    if kind == 1:  # input GEMM of one layer; launch 0 is layer 0
        layer = 0 if plan["regime"] == "wavefront" else launch_index // 2
        il = I if layer == 0 else H
        return 2.0 * G * H * il * B * T
    if kind != 2:  # clearing the step counters
        return 0.0
    if plan["regime"] == "wavefront":  # R h for every layer + the fused W u products
        fused_in = (I + (L - 1) * H) if plan["input_gemms"] == 0 else (L - 1) * H
        return 2.0 * G * H * H * B * T * L + 2.0 * G * H * fused_in * B * T
    return 2.0 * G * H * H * B * T  # layerwise: one layer's recurrence


def kernel_source_digest() -> str:
    """sha256 over the library sources (kernels, planner, launch code): HBM counter
    figures taken for other sources no longer describe the kernel."""
    import hashlib
    csrc = os.path.join(ROOT, "stacked_lstm_forward_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".h", ".hip", ".cpp")):
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


def cpu_baseline(inp, cfg, min_seconds: float) -> dict:
    import numpy as np  # noqa: F401
    from oracle.lstm_oracle import lstm_forward_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    reps, t0 = 0, time.perf_counter()
    while True:
        lstm_forward_inputs(inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 50:
            break
    return {"value": cfg.flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole workload ({cfg.name}) run {reps}x by the fp64 NumPy oracle in {el:.1f} s "
                      f"({el / reps * 1e3:.0f} ms per forward)"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--cell", default="lstm", choices=["lstm", "gru", "rnn_tanh", "rnn_relu"],
                    help="recurrent cell at the workload's shapes (the headline metric is the LSTM)")
    ap.add_argument("--regime", type=int, default=0, help="0 auto, 1 layerwise, 2 wavefront")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (calibrates HBM traffic counters)")
    ap.add_argument("--plain-launch", action="store_true",
                    help="ordinary (not cooperative) launch of the persistent kernel, for profilers")
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
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else 0.5 * (
        per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])

    # per-kernel durations from the library's launch events
    per_kind: dict = {}
    flops_kind: dict = {}
    for k in range(args.steps):
        n = nls[k].value
        for j in range(n):
            kind = kinds[k][j]
            d = evs[k][j].elapsed_time(evs[k][maxl + j])
            per_kind.setdefault(kind, []).append(d)
            flops_kind.setdefault(kind, []).append(kernel_flops(cfg, kind, plan, j))
    dom = max(per_kind, key=lambda kk: sum(per_kind[kk]))
    dom_ms = sum(per_kind[dom]) / len(per_kind[dom])
    dom_flops = sum(flops_kind[dom]) / len(flops_kind[dom])
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    value = cfg.flops / (ms_step * 1e-3) / 1e12
    y, hT, cT = prob.outputs_f32()
    import numpy as np
    if not (np.all(np.isfinite(y)) and np.all(np.isfinite(hT)) and (cT is None or np.all(np.isfinite(cT)))):
        print("non-finite outputs", file=sys.stderr)
        return 1
    log(f"{ms_step:.4f} ms/step, {value:.2f} TFLOP/s; dominant kernel kind {dom}: {dom_ms:.4f} ms/launch")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host (cpu_baseline)")
        cpu = cpu_baseline(inp, cfg, args.cpu_seconds)

    kname = {1: "lstm_input_gemm", 2: "lstm_rec_kernel", 3: "lstm_clear"}
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
        "ms_per_sequence": round(ms_step / cfg.B, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic (seeded: W,R,b ~ U(-1/sqrt(H),1/sqrt(H)), x ~ N(0,1), h0=c0=0)",
        "config": {"workload": workload, "cell": cfg.cell, "L": cfg.L, "I": cfg.I, "H": cfg.H, "B": cfg.B,
                   "T": cfg.T, "regime": plan["regime"], "gflop_per_step": round(cfg.flops / 1e9, 3)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(cfg.name, kname.get(dom, str(dom))),
                     "kernel": kname.get(dom, str(dom)), "ms_per_launch": round(dom_ms, 5),
                     "gflop_per_launch": round(dom_flops / 1e9, 3)},
        "whole_step_frac_of_mfma_peak": round(value / peak, 4),
        "kernels_ms_per_launch": {kname.get(kk, str(kk)): round(sum(v) / len(v), 5) for kk, v in per_kind.items()},
        # every kernel that does arithmetic, not only the dominant one (the
        # input GEMMs and the recurrence of a layerwise run bind differently)
        "kernels_mfma_frac": {
            kname.get(kk, str(kk)): round(sum(flops_kind[kk]) / (sum(v) * 1e-3) / 1e12 / peak, 4)
            for kk, v in per_kind.items() if sum(flops_kind[kk]) > 0},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
