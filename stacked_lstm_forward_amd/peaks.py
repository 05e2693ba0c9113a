"""Measured peaks of the device (binding of ``include/lstm_peaks.h``).

    python -m stacked_lstm_forward_amd.peaks [--steps]

prints one JSON line: the matrix-core rates (bf16 16x16x32 and 32x32x16,
fp32 16x16x4), HBM read and copy rates, the LDS read rate, and with --steps
the latency of one step of the persistent kernels' exchange protocol across
the 8 XCDs and inside one XCD.  ``measure_peaks()`` is what bench.py calls.
Argument marshalling only: the kernels are in ``lib/liblstm_peaks.so``.
"""
from __future__ import annotations

import ctypes
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "liblstm_peaks.so")
EXPORTED = ("lstm_peak_mfma", "lstm_peak_memory", "lstm_peak_lds", "lstm_peak_step_ws_bytes", "lstm_peak_step")

MFMA_FLOPS = {0: 2 * 16 * 16 * 32, 1: 2 * 32 * 32 * 16, 2: 2 * 16 * 16 * 4}
_lib = None


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m stacked_lstm_forward_amd.build`")
    # torch first: it brings its own HIP runtime (soname libamdhip64.so.7),
    # which the library's dependency then resolves to.  Loaded the other way
    # round, the process would hold two HIP runtimes and torch's streams and
    # memory would be foreign to the library's.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.lstm_peak_mfma.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp]
    lib.lstm_peak_mfma.restype = i32
    lib.lstm_peak_memory.argtypes = [i32, vp, sz, i32, vp, i32, vp, vp, vp]
    lib.lstm_peak_memory.restype = i32
    lib.lstm_peak_lds.argtypes = [i32, i32, vp, i32, vp, vp, vp]
    lib.lstm_peak_lds.restype = i32
    lib.lstm_peak_step_ws_bytes.argtypes = [i32, i32, i32, i32]
    lib.lstm_peak_step_ws_bytes.restype = sz
    lib.lstm_peak_step.argtypes = [i32, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp]
    lib.lstm_peak_step.restype = i32
    _lib = lib
    return lib


def _timed(launch, reps: int = 3) -> float:
    """Best of `reps` runs of launch(stream, ev0, ev1) -> status, in ms (one warm-up first)."""
    import torch
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)  # torch creates the HIP events on first record
    e1.record(s)
    torch.cuda.synchronize()
    best = None
    for r in range(reps + 1):
        st = launch(s.cuda_stream, e0.cuda_event, e1.cuda_event)
        if st != 0:
            raise RuntimeError(f"microbenchmark launch failed with status {st}")
        torch.cuda.synchronize()
        if r:
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    return best


def mfma_tflops(kind: int, num_cus: int) -> float:
    import torch
    lib = load_library()
    out = torch.zeros(4, dtype=torch.float32, device="cuda:0")
    grid = num_cus * 8
    iters = 20000 if kind == 0 else 10000
    ms = _timed(lambda s, a, b: lib.lstm_peak_mfma(kind, grid, iters, out.data_ptr(), 0, s, a, b))
    return grid * 4 * iters * 8 * MFMA_FLOPS[kind] / (ms * 1e-3) / 1e12


def memory_gbs(mode: int, nbytes: int = 2 << 30) -> float:
    import torch
    lib = load_library()
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    out = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    ms = _timed(lambda s, a, b: lib.lstm_peak_memory(mode, buf.data_ptr(), nbytes, 4096, out.data_ptr(), 0, s, a, b))
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def lds_gbs(num_cus: int) -> float:
    import torch
    lib = load_library()
    out = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    grid, iters = num_cus * 2, 20000
    ms = _timed(lambda s, a, b: lib.lstm_peak_lds(grid, iters, out.data_ptr(), 0, s, a, b))
    return grid * 256 * iters * 8 * 16 / (ms * 1e-3) / 1e9


def step_latency(grid: int, stride: int, scope: int, slice_bytes: int, steps: int = 2000) -> dict:
    """Microseconds per step of the exchange protocol among grid/stride workgroups."""
    import torch
    lib = load_library()
    n = lib.lstm_peak_step_ws_bytes(grid, stride, slice_bytes, steps)
    if n == 0:
        raise ValueError("bad step-benchmark shape")
    raw = torch.empty(n + 256, dtype=torch.uint8, device="cuda:0")
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + n]
    xcc = torch.full((grid,), -1, dtype=torch.int32, device="cuda:0")
    ms = _timed(lambda s, a, b: lib.lstm_peak_step(grid, stride, scope, slice_bytes, steps, 2000000, ws.data_ptr(),
                                                   xcc.data_ptr(), s, a, b), reps=2)
    err = int(ws[:4].view(torch.int32).item())
    ids = xcc.cpu().tolist()
    active = sorted({ids[i] for i in range(0, grid, stride)})
    return {"workgroups": (grid + stride - 1) // stride, "scope": "agent" if scope == 0 else "xcd-l2",
            "slice_bytes": slice_bytes, "us_per_step": ms * 1e3 / steps, "xcds_of_active": active,
            "valid": err == 0}


def measure_peaks() -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    cus = p.multi_processor_count
    bf16 = {"16x16x32": mfma_tflops(0, cus), "32x32x16": mfma_tflops(1, cus)}
    out = {"mfma_tflops": {"bf16": max(bf16.values()), "f32": mfma_tflops(2, cus)},
           "mfma_bf16_by_shape": bf16,
           "hbm_gbs": memory_gbs(0), "hbm_copy_gbs": memory_gbs(1),
           "lds_gbs": lds_gbs(cus), "num_cus": cus}
    out = {k: ({kk: round(vv, 1) for kk, vv in v.items()} if isinstance(v, dict) else
               (round(v, 1) if isinstance(v, float) else v)) for k, v in out.items()}
    return out


def main() -> int:
    import torch
    if not torch.cuda.is_available():
        print("needs a HIP device", file=sys.stderr)
        return 1
    res = measure_peaks()
    print(json.dumps(res), flush=True)
    if "--steps" in sys.argv:
        cus = res["num_cus"]
        rows = []
        # (grid, stride, scope, slice): workgroups spread over the 8 XCDs (stride 1),
        # or every 8th, which share one XCD (stride 8); slice 0 = counters only
        shapes = [(cus, 1, 0, 0), (cus, 1, 0, 64), (192, 1, 0, 64), (128, 1, 0, 96), (64, 1, 0, 192),
                  (32, 1, 0, 384), (8, 1, 0, 0), (cus, 8, 0, 0), (cus, 8, 0, 384)]
        if "--l2-scope" in sys.argv:  # ordinary stores, L2-level polls (measured invalid: the L1 keeps the line)
            shapes += [(cus, 8, 1, 0)]
        for grid, stride, scope, sl in shapes:
            r = step_latency(grid, stride, scope, sl)
            print(json.dumps(r), flush=True)
            rows.append(r)
    return 0


if __name__ == "__main__":
    sys.exit(main())
