"""Builds the gfx950 shared libraries in-tree with hipcc:

    lib/liblstm_fwd.so    the forward pass (include/lstm_fwd.h)
    lib/liblstm_peaks.so  the measured-peak microbenchmarks (include/lstm_peaks.h)

    python -m stacked_lstm_forward_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "liblstm_fwd.so")
PEAKS_LIB = os.path.join(LIBDIR, "liblstm_peaks.so")
ARCH = "gfx950"
# (source, extra defines): the recurrent kernel is instantiated once per
# (dtype, weight source, waves per workgroup) so the variants compile in parallel
UNITS = [("lstm_kernels.hip", [])] + [
    ("lstm_rec_inst.hip", [f"-DLSTM_INST_BF16={bf}", f"-DLSTM_INST_STREAM={st}", f"-DLSTM_INST_NWV={nwv}"])
    for bf in (0, 1) for st in (0, 1) for nwv in (4, 8)
] + [("lstm_rec_res_inst.hip", [f"-DLSTM_RES_SHAPE={k}"]) for k in range(3)] + [("lstm_fwd.cpp", []), ("lstm_plan.cpp", []), ("lstm_fwd_noalloc.hip", []),
                 ("lstm_bwd.hip", [])] + [
    ("lstm_bwd_res_inst.hip", [f"-DLSTM_BWD_RES_SHAPE={k}"]) for k in range(16)]
PEAK_UNITS = [("lstm_peaks.hip", [])]
BUILD_DIR = os.path.join(HERE, "_build")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # keep hipcc from forming packed fp32 instructions (v_pk_*_f32)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(os.path.dirname(HERE), "include")]


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for tag, units in (("fwd", UNITS), ("peaks", PEAK_UNITS)):
        for i, (src, defs) in enumerate(units):
            obj = os.path.join(BUILD_DIR, f"{tag}_{i:02d}_{os.path.splitext(src)[0]}.o")
            jobs.append((tag, obj, [cc, *_flags(), *defs, "-c", os.path.join(CSRC, src), "-o", obj]))

    def run(job):
        _, obj, cmd = job
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(run, jobs))
    for tag, lib in (("fwd", LIB), ("peaks", PEAKS_LIB)):
        mine = [o for (t, _, _), o in zip(jobs, objs) if t == tag]
        tmp = lib + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *mine, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
