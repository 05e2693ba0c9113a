"""GPU parity of the GRU and simple-RNN cells (desc.cell) against the fp64 oracle.

Same tolerances as the LSTM: max-norm relative error of y and hT, 1e-4 for
fp32 and 2e-2 for bf16 inputs (fp32 arithmetic in both).  Every case prints
its name before touching the GPU.
"""
import numpy as np
import pytest

import lstm_inputs as li
import oracle.lstm_oracle as orc
from tests.parity_log import record
from tests.pins import rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
CELLS = ["gru", "rnn_tanh", "rnn_relu"]


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import stacked_lstm_forward_amd as sl
    sl.load_library()
    return "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_gpu(inp, dev, regime=0):
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    opts = sl.LstmOpts()
    opts.force_regime = regime
    prob = runner.prepare(inp, dev)
    prob.run(opts=opts)
    st = sl.lstm_fwd_last_error(prob.ws)
    assert st == sl.LSTM_OK, sl.lstm_status_string(st)
    y, hT, cT = prob.outputs_f32()
    assert cT is None
    return y, hT


def check(got, ref, tol, what):
    ey, eh = rel_err(got[0], ref[0]), rel_err(got[1], ref[1])
    say(f"{what}: y={ey:.2e} hT={eh:.2e}")
    record(what, tol, {"y": ey, "hT": eh})
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1])), what
    assert ey <= tol and eh <= tol, (what, ey, eh)


TINY = [(1, 1, 1, 1, 1), (1, 3, 5, 2, 3), (2, 7, 9, 3, 5), (3, 33, 17, 17, 4), (2, 64, 64, 16, 6),
        (2, 40, 72, 33, 5), (2, 129, 257, 5, 3)]


@pytest.mark.parametrize("regime", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", TINY)
@pytest.mark.parametrize("cell", CELLS)
def test_cells_tiny_shapes(dev, cell, shape, dtype, regime):
    L, I, H, B, T = shape
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=300 + L + I + H, cell=cell)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"{cell} tiny {shape} {dtype} regime={regime}")
    got = run_gpu(inp, dev, regime)
    check(got, orc.forward_inputs(inp)[:2], TOL[dtype], f"{cell} tiny {shape} {dtype} r{regime}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
@pytest.mark.parametrize("cell", CELLS)
def test_cells_workload_shapes(dev, cell, name):
    cfg = li.with_cell(li.CONFIGS[name], cell)
    inp = li.make_inputs(cfg)
    say(f"{cell} at workload {name} shapes")
    got = run_gpu(inp, dev)
    check(got, orc.forward_inputs(inp)[:2], TOL[cfg.dtype], f"{cell} {name}")


@pytest.mark.parametrize("cell", CELLS)
def test_cells_large_hidden(dev, cell):
    """c4 shapes (H = 4096, recurrent weights in registers and LDS), T = 12:
    every sequence of the batch against the oracle."""
    cfg = li.with_cell(li.CONFIGS["c4"], cell)
    cfg = li.Config(cfg.name + "-T12", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, 12, cfg.dtype, cell)
    inp = li.make_inputs(cfg)
    say(f"{cell} at c4 shapes, T=12, all 32 sequences")
    got = run_gpu(inp, dev)
    check(got, orc.forward_inputs(inp)[:2], TOL[cfg.dtype], f"{cell} c4 T12")


@pytest.mark.parametrize("cell", CELLS)
def test_cells_regimes_agree(dev, cell):
    cfg = li.with_cell(li.CONFIGS["c2"], cell)
    cfg = li.Config(cfg.name + "-T16", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, 16, cfg.dtype, cell)
    inp = li.make_inputs(cfg, random_state=True)
    say(f"{cell} regimes")
    ref = orc.forward_inputs(inp)[:2]
    check(run_gpu(inp, dev, 1), ref, TOL[cfg.dtype], f"{cell} layerwise")
    check(run_gpu(inp, dev, 2), ref, TOL[cfg.dtype], f"{cell} wavefront")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("regime", [1, 2])
def test_gru_open_update_gate_carries_h_bit_exactly(dev, dtype, regime):
    """b_z = +1e4 saturates z to 1: h_t equals h0 bit for bit in every layer and step."""
    L, I, H, B, T = 2, 24, 20, 5, 6
    rng = np.random.default_rng(12)
    W = [rng.uniform(-0.5, 0.5, (3 * H, I if l == 0 else H)) for l in range(L)]
    R = [rng.uniform(-0.5, 0.5, (3 * H, H)) for _ in range(L)]
    b = [rng.uniform(-0.5, 0.5, 4 * H) for _ in range(L)]
    for bl in b:
        bl[H:2 * H] = 1e4
    x = rng.standard_normal((T, B, I))
    h0 = rng.uniform(-1, 1, (L, B, H))
    inp = li.from_arrays(L, I, H, B, T, dtype, x, W, R, b, h0, None, cell="gru")
    say(f"gru saturated update gate {dtype} regime={regime}")
    y, hT = run_gpu(inp, dev, regime)
    h0s = inp.h0_f32()
    assert np.array_equal(hT, h0s)
    assert np.array_equal(y, np.broadcast_to(h0s[-1], y.shape))
