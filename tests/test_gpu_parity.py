"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances (max-norm relative error per output tensor, ||a - r|| / ||r||):
1e-4 for fp32 workloads and 2e-2 for bf16 workloads (fp32 accumulation and
cell state in both).  Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest

import lstm_inputs as li
import oracle.lstm_oracle as orc
from tests.parity_log import record
from tests.pins import rel_err, saturating_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import stacked_lstm_forward_amd as sl
    sl.load_library()
    return "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_gpu(inp, dev, regime=0, timeout_us=0):
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    opts = sl.LstmOpts()
    opts.force_regime = regime
    opts.wait_timeout_us = timeout_us
    prob = runner.prepare(inp, dev)
    prob.run(opts=opts)
    st = sl.lstm_fwd_last_error(prob.ws)
    assert st == sl.LSTM_OK, sl.lstm_status_string(st)
    return prob.outputs_f32()


def check_close(got, ref, tol, what):
    names = ("y", "hT", "cT")
    errs = {n: rel_err(g, r) for n, g, r in zip(names, got, ref)}
    say(f"{what}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    record(what, tol, errs)
    for n in names:
        assert np.all(np.isfinite(got[names.index(n)])), (what, n)
        assert errs[n] <= tol, (what, n, errs[n])
    return errs


# ----------------------------------------------------------------------------- tiny / ragged shapes
TINY = [
    # L, I, H, B, T
    (1, 1, 1, 1, 1),
    (1, 3, 5, 2, 3),
    (2, 7, 9, 3, 5),
    (3, 33, 17, 17, 4),
    (2, 64, 64, 16, 6),
    (1, 130, 66, 20, 7),
    (4, 40, 72, 33, 5),
    (2, 129, 257, 5, 3),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", TINY)
@pytest.mark.parametrize("regime", [1, 2])
def test_tiny_shapes(dev, shape, dtype, regime):
    L, I, H, B, T = shape
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=100 + L + I + H)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"tiny {shape} {dtype} regime={regime}")
    got = run_gpu(inp, dev, regime=regime)
    ref = orc.lstm_forward_inputs(inp)
    check_close(got, ref, TOL[dtype], f"tiny {shape} {dtype} r{regime}")


# ----------------------------------------------------------------------------- load-order exchange
# Aligned shapes (H a multiple of the chunk width) with B >= 16 exchange h in
# load order: ragged last column tile (B = 40), layerwise runs whose next layer's
# input GEMM reads the row-major copy, a wavefront of 18 layers in two launches
# (layer 16 reads layer 15's load-order buffer), and B = 8, which keeps the
# row-major exchange on the aligned path.
ALIGNED = [
    # L, I, H, B, T
    (3, 64, 128, 40, 5),
    (2, 96, 64, 16, 4),
    (18, 32, 64, 16, 3),
    (2, 64, 128, 8, 5),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ALIGNED)
@pytest.mark.parametrize("regime", [1, 2])
def test_aligned_exchange(dev, shape, dtype, regime):
    L, I, H, B, T = shape
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=200 + L + B)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"aligned {shape} {dtype} regime={regime}")
    got = run_gpu(inp, dev, regime=regime)
    ref = orc.lstm_forward_inputs(inp)
    check_close(got, ref, TOL[dtype], f"aligned {shape} {dtype} r{regime}")


# ----------------------------------------------------------------------------- direct-to-LDS input GEMM
# K >= 1024 with aligned rows takes the 256 x 256 direct-to-LDS GEMM: a partial
# M-block (H = 40: 10 M-tiles of 16), a ragged column tile (T * B = 15) and,
# for the GRU, rows without input weights dropped in its epilogue.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cell", ["lstm", "gru"])
def test_input_gemm_direct_to_lds_ragged(dev, dtype, cell):
    cfg = li.custom_config(1, 1024, 40, 3, 5, dtype, cfg_id=61, cell=cell)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"input GEMM K=1024 H=40 B=3 T=5 {dtype} {cell}")
    got = run_gpu(inp, dev)
    ref = orc.forward_inputs(inp)
    if cell != "lstm":
        got, ref = got[:2] + (None,), ref[:2] + (None,)
    names = ("y", "hT", "cT")
    for n, g, r in zip(names, got, ref):
        if r is None:
            continue
        e = rel_err(g, r)
        say(f"  {n}={e:.2e}")
        assert np.all(np.isfinite(g)) and e <= TOL[dtype], (cell, dtype, n, e)


# ----------------------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_workload_full(dev, name):
    cfg = li.CONFIGS[name]
    inp = li.make_inputs(cfg)
    say(f"workload {name} full")
    got = run_gpu(inp, dev)
    ref = orc.lstm_forward_inputs(inp)
    check_close(got, ref, TOL[cfg.dtype], f"workload {name}")


def test_workload_c4_full(dev):
    """H = 4096 (recurrent weights in registers and LDS): every sequence of the
    batch against the oracle."""
    cfg = li.CONFIGS["c4"]
    inp = li.make_inputs(cfg)
    say("workload c4 full (all 32 sequences)")
    got = run_gpu(inp, dev)
    ref = orc.lstm_forward_inputs(inp)
    check_close(got, ref, TOL[cfg.dtype], "workload c4")


@pytest.mark.parametrize("name", ["c1", "c3"])
def test_workload_random_initial_state(dev, name):
    cfg = li.CONFIGS[name]
    inp = li.make_inputs(cfg, random_state=True)
    say(f"workload {name} with random h0/c0")
    got = run_gpu(inp, dev)
    ref = orc.lstm_forward_inputs(inp)
    check_close(got, ref, TOL[cfg.dtype], f"workload {name} h0/c0")


# ----------------------------------------------------------------------------- schedules agree
@pytest.mark.parametrize("name", ["c2", "c3"])
def test_regimes_agree(dev, name):
    cfg = li.CONFIGS[name]
    cfg = li.Config(cfg.name + "-T24", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, 24, cfg.dtype)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"regimes {name}")
    a = run_gpu(inp, dev, regime=1)
    b = run_gpu(inp, dev, regime=2)
    ref = orc.lstm_forward_inputs(inp)
    check_close(a, ref, TOL[cfg.dtype], f"{name} layerwise")
    check_close(b, ref, TOL[cfg.dtype], f"{name} wavefront")


# ----------------------------------------------------------------------------- determinism
@pytest.mark.parametrize("name,regime", [("c3", 0), ("c2", 0), ("c5", 0), ("c3", 1)])
def test_bitwise_deterministic(dev, name, regime):
    import torch
    from stacked_lstm_forward_amd import runner
    import stacked_lstm_forward_amd as sl
    cfg = li.CONFIGS[name]
    if cfg.T > 256:
        cfg = li.Config(cfg.name + "-T256", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, 256, cfg.dtype)
    inp = li.make_inputs(cfg)
    say(f"determinism {name} regime={regime}")
    opts = sl.LstmOpts()
    opts.force_regime = regime
    prob = runner.prepare(inp, dev)
    prob.run(opts=opts)
    first = [t.clone() for t in (prob.y, prob.hT, prob.cT)]
    for _ in range(2):
        prob.ws.fill_(0xA5)  # workspace contents on entry must not matter
        prob.run(opts=opts)
        for a, b in zip(first, (prob.y, prob.hT, prob.cT)):
            assert torch.equal(_bits(a), _bits(b))


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# ----------------------------------------------------------------------------- one workspace, new inputs
# Exchange slots are read with ordinary loads once their step counter is seen;
# that is safe only if no cache can still hold the slot's bits from an earlier
# call on the same workspace.  Two calls with different inputs on one
# workspace: the second must match the oracle for its own inputs.
BACK_TO_BACK = [
    # name, L, I, H, B, T, dtype, regime: wavefront, layerwise, register-resident
    ("wavefront", 3, 128, 256, 64, 12, "bf16", 2),
    ("layerwise", 2, 512, 512, 64, 10, "f32", 1),
    ("layerwise-B4", 1, 256, 1536, 4, 40, "bf16", 1),
    ("resident", 1, 512, 4096, 32, 6, "bf16", 0),
]


@pytest.mark.parametrize("name,L,I,H,B,T,dtype,regime", BACK_TO_BACK)
def test_gpu_same_workspace_new_inputs(dev, name, L, I, H, B, T, dtype, regime):
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    cfg_a = li.custom_config(L, I, H, B, T, dtype, cfg_id=601)
    cfg_b = li.custom_config(L, I, H, B, T, dtype, cfg_id=602)
    inp_a = li.make_inputs(cfg_a, random_state=True)
    inp_b = li.make_inputs(cfg_b, random_state=True)
    if name == "resident":
        assert sl.lstm_fwd_plan(sl.make_desc(L, I, H, B, T, dtype)).weight_blocks_in_registers > 0
    say(f"same workspace, new inputs: {name}")
    a = runner.prepare(inp_a, dev)
    b = runner.prepare(inp_b, dev)
    opts = sl.LstmOpts()
    opts.force_regime = regime
    for prob in (a, b, a, b):  # a's results sit in the workspace (and caches) when b runs
        st = sl.lstm_fwd_ex(prob.desc, prob.x, prob.h0, prob.c0, prob.W, prob.R, prob.b, prob.y, prob.hT, prob.cT,
                            a.ws, None, opts)
        assert st == sl.LSTM_OK
    assert sl.lstm_fwd_last_error(a.ws) == sl.LSTM_OK
    check_close(b.outputs_f32(), orc.lstm_forward_inputs(inp_b), TOL[dtype], f"same ws {name} (second inputs)")
    check_close(a.outputs_f32(), orc.lstm_forward_inputs(inp_a), TOL[dtype], f"same ws {name} (first inputs)")


# ----------------------------------------------------------------------------- pins on the GPU
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpu_saturation_keeps_c_bit_exact(dev, dtype):
    """Forget bias +1e4 and input bias -1e4: cT must equal c0 bit for bit."""
    x, W, R, b, h0, c0 = saturating_inputs(L=2, I=40, H=36, B=5, T=9)
    inp = li.from_arrays(2, 40, 36, 5, 9, dtype, x, W, R, b, h0, c0)
    say(f"saturation {dtype}")
    for regime in (1, 2):
        y, hT, cT = run_gpu(inp, dev, regime=regime)
        assert np.array_equal(cT.view(np.uint32), inp.c0.view(np.uint32)), regime
        ratio = hT / np.tanh(inp.c0_f32())
        assert np.all(ratio >= 0) and np.all(ratio <= 1.0 + 1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpu_zero_bias_zero_state_stays_zero(dev, dtype):
    """x = 0, R arbitrary, b = 0, h0 = c0 = 0: h and c stay exactly 0."""
    L, I, H, B, T = 2, 24, 20, 3, 6
    rng = np.random.default_rng(1)
    W = [rng.uniform(-1, 1, (4 * H, I if l == 0 else H)) for l in range(L)]
    R = [rng.uniform(-1, 1, (4 * H, H)) for l in range(L)]
    b = [np.zeros(4 * H) for _ in range(L)]
    inp = li.from_arrays(L, I, H, B, T, dtype, np.zeros((T, B, I)), W, R, b)
    say(f"zero state {dtype}")
    y, hT, cT = run_gpu(inp, dev)
    assert np.all(y == 0) and np.all(hT == 0) and np.all(cT == 0)


def test_gpu_zero_recurrence_closed_form(dev):
    """Zero x and zero R: c_t = c* + f^t (c0 - c*) per unit (fp32)."""
    L, I, H, B, T = 1, 8, 12, 3, 16
    rng = np.random.default_rng(4)
    W = [rng.uniform(-1, 1, (4 * H, I))]
    R = [np.zeros((4 * H, H))]
    b = [rng.uniform(-1.5, 1.5, 4 * H)]
    c0 = rng.uniform(-1, 1, (1, B, H))
    inp = li.from_arrays(L, I, H, B, T, "f32", np.zeros((T, B, I)), W, R, b, None, c0)
    say("zero recurrence closed form")
    y, hT, cT = run_gpu(inp, dev)
    bb = inp.b_f32(0).astype(np.float64)
    sg = lambda z: 1 / (1 + np.exp(-z))  # noqa: E731
    i, f, g, o = sg(bb[:H]), sg(bb[H:2 * H]), np.tanh(bb[2 * H:3 * H]), sg(bb[3 * H:])
    cstar = i * g / (1 - f)
    c0v = inp.c0_f32().astype(np.float64)[0]
    ct = cstar + f ** T * (c0v - cstar)
    assert rel_err(cT[0], ct) < 1e-5
    assert rel_err(y[-1], o * np.tanh(ct)) < 1e-5


# ----------------------------------------------------------------------------- resume from (hT, cT)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpu_time_split_resume(dev, dtype):
    L, I, H, B, T, T1 = 3, 48, 64, 9, 12, 5
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=321)
    full = li.make_inputs(cfg, random_state=True)
    say(f"time split {dtype}")
    y, hT, cT = run_gpu(full, dev, regime=1)
    a = li.Inputs(li.custom_config(L, I, H, B, T1, dtype), full.x[:T1], full.W, full.R, full.b, full.h0, full.c0)
    ya, ha, ca = run_gpu(a, dev, regime=1)
    h_bits = li.to_storage(ha, dtype) if dtype == "f32" else li.bf16_bits_from_f32(ha)
    bpart = li.Inputs(li.custom_config(L, I, H, B, T - T1, dtype), full.x[T1:], full.W, full.R, full.b,
                      h_bits, ca.astype(np.float32))
    yb, hb, cb = run_gpu(bpart, dev, regime=1)
    assert np.array_equal(np.concatenate([ya, yb]), y)
    assert np.array_equal(hb, hT) and np.array_equal(cb, cT)


# ----------------------------------------------------------------------------- outputs optional, errors
def test_gpu_null_final_states(dev):
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    cfg = li.custom_config(2, 16, 32, 4, 5, "f32", cfg_id=77)
    inp = li.make_inputs(cfg)
    say("null hT/cT")
    prob = runner.prepare(inp, dev)
    st = sl.lstm_fwd(prob.desc, prob.x, None, None, prob.W, prob.R, prob.b, prob.y, None, None, prob.ws)
    assert st == sl.LSTM_OK
    assert sl.lstm_fwd_last_error(prob.ws) == sl.LSTM_OK
    ref = orc.lstm_forward_inputs(inp)
    assert rel_err(prob.y.float().cpu().numpy(), ref[0]) < TOL["f32"]


def test_gpu_forced_wait_timeout_reports_error(dev):
    """A negative wait limit fails every blocked step wait at once: the kernel
    exits normally and the error word reports the timeout; the next call is clean."""
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    cfg = li.custom_config(3, 32, 64, 8, 6, "bf16", cfg_id=78)
    inp = li.make_inputs(cfg)
    prob = runner.prepare(inp, dev)
    for regime in (1, 2):
        say(f"forced timeout regime={regime}")
        opts = sl.LstmOpts()
        opts.force_regime = regime
        opts.wait_timeout_us = -1
        prob.run(opts=opts)
        assert sl.lstm_fwd_last_error(prob.ws) == sl.LSTM_ERR_BARRIER_TIMEOUT
    prob.run()
    assert sl.lstm_fwd_last_error(prob.ws) == sl.LSTM_OK
    ref = orc.lstm_forward_inputs(inp)
    assert rel_err(prob.y.float().cpu().numpy(), ref[0]) < TOL["bf16"]


def test_gpu_launch_events(dev):
    """lstm_fwd_ex records one event pair per launch and reports each kind."""
    import ctypes
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    cfg = li.CONFIGS["c3"]
    cfg = li.Config("c3-T8", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, 8, cfg.dtype)
    inp = li.make_inputs(cfg)
    prob = runner.prepare(inp, dev)
    say("launch events")
    n = 16
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for e in evs:  # torch creates the HIP event on first record
        e.record()
    torch.cuda.synchronize()
    start = (ctypes.c_void_p * n)(*[e.cuda_event for e in evs[:n]])
    stop = (ctypes.c_void_p * n)(*[e.cuda_event for e in evs[n:]])
    kinds = (ctypes.c_int32 * n)()
    nl = ctypes.c_int32(0)
    opts = sl.LstmOpts()
    opts.max_launches = n
    opts.ev_start = ctypes.cast(start, ctypes.POINTER(ctypes.c_void_p))
    opts.ev_stop = ctypes.cast(stop, ctypes.POINTER(ctypes.c_void_p))
    opts.launch_kind = kinds
    opts.num_launches = ctypes.pointer(nl)
    prob.run(opts=opts)
    torch.cuda.synchronize()
    plan = sl.lstm_fwd_plan(prob.desc).as_dict()
    first = sl.LSTM_KERNEL_INPUT_GEMM if plan["input_gemms"] else sl.LSTM_KERNEL_CLEAR
    assert nl.value == plan["num_launches"] == 2
    assert list(kinds[:2]) == [first, sl.LSTM_KERNEL_RECURRENT]
    for k in range(2):
        assert evs[k].elapsed_time(evs[n + k]) > 0
    # layerwise: input GEMM then recurrence, per layer
    opts.force_regime = 1
    prob.run(opts=opts)
    torch.cuda.synchronize()
    assert nl.value == 2 * cfg.L
    assert list(kinds[:nl.value]) == [sl.LSTM_KERNEL_INPUT_GEMM, sl.LSTM_KERNEL_RECURRENT] * cfg.L


def test_gpu_wavefront_with_hoisted_first_layer(dev):
    """A first layer too wide to keep [W_0 | R_0] on chip: the wavefront hoists its
    input product into the input GEMM and fuses only the layers above."""
    import stacked_lstm_forward_amd as sl
    cfg = li.custom_config(2, 4096, 16, 4, 3, "f32", cfg_id=79)
    inp = li.make_inputs(cfg, random_state=True)
    say("wavefront with hoisted layer 0 (I=4096, H=16)")
    d = sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype)
    plan = sl.lstm_fwd_plan(d, 2).as_dict()
    assert plan["regime"] == "wavefront" and plan["input_gemms"] == 1
    got = run_gpu(inp, dev, regime=2)
    check_close(got, orc.lstm_forward_inputs(inp), TOL["f32"], "wavefront hoisted layer 0")


# ----------------------------------------------------------------------------- counter-free exchange
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,B", [(128, 8), (256, 4)])
def test_gpu_data_valid_exchange_parity(dev, H, B, dtype):
    """Small single-layer grids exchange h_t without step counters (readers re-read
    the slot until no element holds the unwritten pattern): same results."""
    import stacked_lstm_forward_amd as sl
    cfg = li.custom_config(2, H, H, B, 40, dtype, cfg_id=90)
    d = sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype)
    assert sl.lstm_fwd_plan(d, 1).as_dict()["data_valid_exchange"]
    inp = li.make_inputs(cfg, random_state=True)
    say(f"data-valid exchange H={H} B={B} {dtype}")
    check_close(run_gpu(inp, dev, regime=1), orc.lstm_forward_inputs(inp), TOL[dtype], f"dv H{H} B{B} {dtype}")


def test_gpu_data_valid_exchange_forced_timeout(dev):
    """A zero wait limit makes the first incomplete re-read give up: every workgroup
    leaves the kernel, the error word reports the timeout and the next call is clean."""
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    cfg = li.custom_config(2, 256, 256, 8, 6, "bf16", cfg_id=91)
    d = sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype)
    assert sl.lstm_fwd_plan(d, 1).as_dict()["data_valid_exchange"]
    inp = li.make_inputs(cfg)
    prob = runner.prepare(inp, dev)
    say("data-valid exchange forced timeout")
    opts = sl.LstmOpts()
    opts.force_regime = 1
    opts.wait_timeout_us = -1
    prob.run(opts=opts)
    assert sl.lstm_fwd_last_error(prob.ws) == sl.LSTM_ERR_BARRIER_TIMEOUT
    prob.run()
    assert sl.lstm_fwd_last_error(prob.ws) == sl.LSTM_OK
    ref = orc.lstm_forward_inputs(inp)
    assert rel_err(prob.y.float().cpu().numpy(), ref[0]) < TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpu_data_valid_exchange_nan_input(dev, dtype):
    """An input element with every bit set (a NaN, and the exchange's unwritten
    pattern) makes that sequence's h NaN from then on; stored NaNs are canonical,
    so no reader mistakes them for unwritten slots and the call ends normally."""
    import warnings
    import dataclasses
    import stacked_lstm_forward_amd as sl
    cfg = li.custom_config(1, 128, 128, 8, 5, dtype, cfg_id=92)
    d = sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype)
    assert sl.lstm_fwd_plan(d, 0).as_dict()["data_valid_exchange"]
    inp = li.make_inputs(cfg)
    x = inp.x.copy()
    if dtype == "bf16":
        x[1, 0, 3] = 0xFFFF
    else:
        x.view(np.uint32)[1, 0, 3] = 0xFFFFFFFF
    inp = dataclasses.replace(inp, x=x)
    say(f"all-ones NaN input {dtype}")
    got = run_gpu(inp, dev)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        ref = orc.lstm_forward_inputs(inp)
    for g, r, what in zip(got, ref, ("y", "hT", "cT")):
        assert np.array_equal(np.isnan(g), np.isnan(r)), what
        fin = ~np.isnan(r)
        assert np.isnan(r).any() and fin.any(), what
        err = np.max(np.abs(g[fin] - r[fin])) / np.max(np.abs(r[fin]))
        assert err <= TOL[dtype], (what, err)


# ----------------------------------------------------------------------------- size limits
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("regime", [1, 2])
@pytest.mark.parametrize("shape", [(64, 32, 32, 4, 3), (2, 64, 64, 256, 3)])
def test_gpu_size_limits(dev, shape, dtype, regime):
    """The largest stack (64 layers: four 16-layer wavefront launches) and the
    largest batch (256 = 16 column tiles) the library accepts."""
    L, I, H, B, T = shape
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=95 + L)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"limits {shape} {dtype} regime={regime}")
    got = run_gpu(inp, dev, regime=regime)
    ref = orc.lstm_forward_inputs(inp)
    check_close(got, ref, TOL[dtype], f"limits {shape} {dtype} r{regime}")


@pytest.mark.parametrize("shape,dtype", [((2, 64, 64, 80, 4), "f32"), ((2, 192, 192, 80, 4), "bf16"),
                                         ((3, 128, 128, 48, 4), "bf16")])
def test_gpu_wavefront_padding_tiles(dev, shape, dtype):
    """Two-waves-per-SIMD launches multiply every tile of their instantiation
    without branches: here a wave owns 3 column tiles of a 4-wide instantiation
    (B = 48, 80), and with B = 80 one tile group's third tile is past the batch.
    Those tiles' sums must never reach the outputs."""
    import stacked_lstm_forward_amd as sl
    L, I, H, B, T = shape
    d = sl.make_desc(L, I, H, B, T, dtype)
    plan = sl.lstm_fwd_plan(d, 2).as_dict()
    assert plan["block"] == 512 and plan["wave_tiles"][1] == 3, plan
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=97)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"padding tiles {shape} {dtype}")
    check_close(run_gpu(inp, dev, regime=2), orc.lstm_forward_inputs(inp), TOL[dtype], f"pad {shape} {dtype}")
