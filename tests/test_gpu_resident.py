"""GPU parity of the register-resident recurrent kernel: layers whose recurrent
weights do not fit in LDS but do fit in LDS plus registers stay on chip for the
whole sequence (bf16 H = 4096: 128 MiB; bf16 H = 3072: 72 MiB; fp32 H = 2048:
64 MiB), with up to four 16-column batch tiles.

Every batch column is compared with the oracle (a lane-dependent indexing
mistake in the load-order exchange would show in some column); the same
tolerance as every bf16 workload: max-norm relative error 2e-2 per output.
Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest

import lstm_inputs as li
import oracle.lstm_oracle as orc
from tests.parity_log import record
from tests.pins import rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_F32 = 1e-4


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import stacked_lstm_forward_amd as sl
    sl.load_library()
    return "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def resident_plan(cfg):
    import stacked_lstm_forward_amd as sl
    d = sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype, cfg.cell)
    return sl.lstm_fwd_plan(d, 0, 0, 0)


def run(inp, dev):
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    prob = runner.prepare(inp, dev)
    prob.run()
    st = sl.lstm_fwd_last_error(prob.ws)
    assert st == sl.LSTM_OK, sl.lstm_status_string(st)
    return prob


def check(got, ref, what, tol=TOL):
    names = ("y", "hT", "cT")
    errs = {}
    for n, g, r in zip(names, got, ref):
        if r is None:
            assert g is None
            continue
        assert np.all(np.isfinite(g)), (what, n)
        errs[n] = rel_err(g, r)
    say(f"{what}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    record(what, tol, errs)
    for n, e in errs.items():
        assert e <= tol, (what, n, e)


# B = 16: one column tile; 20: a ragged second tile; 32: two full tiles
@pytest.mark.parametrize("B", [16, 20, 32])
@pytest.mark.parametrize("random_state", [False, True])
def test_gpu_resident_lstm(dev, B, random_state):
    cfg = li.custom_config(1, 256, 4096, B, 4, "bf16", cfg_id=310 + B)
    info = resident_plan(cfg)
    assert info.weight_blocks_in_registers == 48 and info.weights_on_chip and not info.weights_streamed
    inp = li.make_inputs(cfg, random_state=random_state)
    say(f"resident lstm H=4096 B={B} random_state={random_state}")
    got = run(inp, dev).outputs_f32()
    ref = orc.forward_inputs(inp)
    check(got, ref, f"resident lstm B={B} rs={int(random_state)}")
    # per column as well: every batch lane of both column tiles
    for col in range(B):
        e = max(rel_err(g[:, col], r[:, col]) for g, r in zip(got, ref))
        assert e <= TOL, (B, col, e)


def test_gpu_resident_gru(dev):
    cfg = li.with_cell(li.custom_config(1, 256, 4096, 32, 3, "bf16", cfg_id=341), "gru")
    assert resident_plan(cfg).weight_blocks_in_registers == 48
    inp = li.make_inputs(cfg, random_state=True)
    say("resident gru H=4096 B=32")
    y, hT, cT = run(inp, dev).outputs_f32()
    ref = orc.forward_inputs(inp)
    check((y, hT, None), ref, "resident gru")


def test_gpu_resident_two_layers_deterministic(dev):
    """Two resident layers in a row (layer 1 reads layer 0's exchange buffer),
    and three calls give the same bits whatever the workspace held."""
    import torch
    cfg = li.custom_config(2, 128, 4096, 24, 3, "bf16", cfg_id=342)
    assert resident_plan(cfg).weight_blocks_in_registers == 48
    inp = li.make_inputs(cfg, random_state=True)
    say("resident two layers H=4096 B=24, determinism")
    prob = run(inp, dev)
    first = [t.clone() for t in (prob.y, prob.hT, prob.cT)]
    ref = orc.forward_inputs(inp)
    check(prob.outputs_f32(), ref, "resident two layers")
    for _ in range(2):
        prob.ws.fill_(0x5A)
        prob.run()
        for a, b in zip(first, (prob.y, prob.hT, prob.cT)):
            va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
            vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
            assert torch.equal(va, vb)


def per_column(got, ref, B, tol, what):
    for col in range(B):
        e = max(rel_err(g[:, col], r[:, col]) for g, r in zip(got, ref))
        assert e <= tol, (what, col, e)


# three and four column tiles (48 and 64 sequences; 40: a ragged third tile)
@pytest.mark.parametrize("B", [40, 48, 64])
def test_gpu_resident_lstm_wide_batch(dev, B):
    cfg = li.custom_config(1, 256, 4096, B, 3, "bf16", cfg_id=350 + B)
    info = resident_plan(cfg)
    assert info.weight_blocks_in_registers == 48 and info.weights_on_chip and not info.weights_streamed
    inp = li.make_inputs(cfg, random_state=True)
    say(f"resident lstm H=4096 B={B}")
    got = run(inp, dev).outputs_f32()
    ref = orc.forward_inputs(inp)
    check(got, ref, f"resident lstm H4096 B={B}")
    per_column(got, ref, B, TOL, f"H4096 B={B}")


# the other resident shapes: bf16 H = 3072 (all 36 blocks of a wave in
# registers) and fp32 H = 2048 (16 in registers, 16 in LDS)
@pytest.mark.parametrize("H,dtype,nrb,B", [(3072, "bf16", 36, 16), (3072, "bf16", 36, 32), (3072, "bf16", 36, 52),
                                           (2048, "f32", 16, 8), (2048, "f32", 16, 32)])
def test_gpu_resident_other_shapes(dev, H, dtype, nrb, B):
    cfg = li.custom_config(1, 192, H, B, 4, dtype, cfg_id=370 + B + H // 1024)
    info = resident_plan(cfg)
    assert info.weight_blocks_in_registers == nrb and info.weights_on_chip and not info.weights_streamed
    inp = li.make_inputs(cfg, random_state=True)
    say(f"resident lstm H={H} {dtype} B={B}")
    got = run(inp, dev).outputs_f32()
    ref = orc.forward_inputs(inp)
    tol = TOL if dtype == "bf16" else TOL_F32
    check(got, ref, f"resident lstm H{H} {dtype} B={B}", tol)
    per_column(got, ref, B, tol, f"H{H} {dtype} B={B}")


def test_gpu_resident_two_layers_h3072(dev):
    """Two stacked H = 3072 layers, the second reading the first's row-major copy."""
    cfg = li.custom_config(2, 3072, 3072, 32, 3, "bf16", cfg_id=390)
    assert resident_plan(cfg).weight_blocks_in_registers == 36
    inp = li.make_inputs(cfg, random_state=True)
    say("resident two layers H=3072 B=32")
    got = run(inp, dev).outputs_f32()
    check(got, orc.forward_inputs(inp), "resident two layers H3072")
