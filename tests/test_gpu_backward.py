"""GPU parity of the training passes: lstm_fwd_train (the forward that keeps
gates, cell and hidden states) and lstm_bwd (backpropagation through time)
against the fp64 backward oracle, through the C ABI.

Every gradient tensor (dx, dh0, dc0, and per layer dW, dR, db) must be within
the workload dtype's max-norm relative tolerance of the oracle: 1e-4 for fp32,
2e-2 for bf16 (whose products take bf16 operands, like its forward).  The
training forward's outputs must equal lstm_fwd's bit for bit.  Every case
prints its name before touching the GPU.
"""
import numpy as np
import pytest

import lstm_inputs as li
import oracle.lstm_oracle_bwd as orcb
from tests.parity_log import record
from tests.pins import rel_err

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


def upstream(cfg, seed, with_states=True):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((cfg.T, cfg.B, cfg.H))
    if not with_states:
        return dy, None, None
    return dy, rng.standard_normal((cfg.L, cfg.B, cfg.H)), rng.standard_normal((cfg.L, cfg.B, cfg.H))


def run_and_check(inp, dy, dhT, dcT, dev, what):
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    tp = runner.prepare_train(inp, dy, dhT, dcT, dev)
    tp.forward()
    assert sl.lstm_fwd_last_error(tp.fwd.ws) == sl.LSTM_OK
    ref_fwd = runner.prepare(inp, dev)
    ref_fwd.run()
    for a, b in zip((tp.fwd.y, tp.fwd.hT, tp.fwd.cT), (ref_fwd.y, ref_fwd.hT, ref_fwd.cT)):
        va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
        vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
        assert torch.equal(va, vb), "training forward must equal lstm_fwd"
    tp.backward()
    assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_OK
    got = tp.grads_f64()
    # the oracle sees the upstream gradients the GPU saw (rounded to fp32)
    f32 = lambda a: None if a is None else np.asarray(a, dtype=np.float32).astype(np.float64)  # noqa: E731
    ref = orcb.lstm_backward_inputs(inp, f32(dy), f32(dhT), f32(dcT))
    tol = TOL[inp.cfg.dtype]
    errs = {k: rel_err(got[k], ref[k]) for k in ("dx", "dh0", "dc0")}
    for k in ("dW", "dR", "db"):
        errs[k] = max(rel_err(g, r) for g, r in zip(got[k], ref[k]))
    say(f"{what}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    record(what, tol, errs)
    for k, v in errs.items():
        assert np.isfinite(v) and v <= tol, (what, k, v)


SHAPES = [
    # L, I, H, B, T
    (1, 1, 1, 1, 1),
    (1, 3, 5, 2, 3),
    (2, 24, 20, 3, 5),
    (3, 33, 17, 17, 4),
    (2, 64, 64, 16, 6),
    (2, 130, 66, 20, 7),
    (1, 64, 256, 80, 4),  # more than 64 sequences: the streamed chain at a size the on-chip one takes up to B = 64
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
def test_gpu_backward_small(dev, shape, dtype):
    L, I, H, B, T = shape
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=800 + L + I + H)
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 801 + H)
    say(f"backward {shape} {dtype}")
    run_and_check(inp, dy, dhT, dcT, dev, f"bwd {shape} {dtype}")


@pytest.mark.parametrize("name,T", [("c1", None), ("c2", None), ("c3", None), ("c5", None)])
def test_gpu_backward_workload_shapes(dev, name, T):
    """The workloads in full (every step; the fp64 oracle takes about 25 s for
    c5's 2048 steps), zero initial states, dy only."""
    import stacked_lstm_forward_amd as sl
    cfg = li.CONFIGS[name]
    if T is not None:
        cfg = li.Config(f"{cfg.name}-T{T}", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, T, cfg.dtype)
    # every workload runs the chain on chip
    assert sl.lstm_bwd_chain_on_chip(sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype))
    inp = li.make_inputs(cfg)
    dy, _, _ = upstream(cfg, 810, with_states=False)
    say(f"backward workload {cfg.name}")
    run_and_check(inp, dy, None, None, dev, f"bwd {cfg.name}")


def test_gpu_backward_large_hidden(dev):
    """H = 4096 (the forward keeps R in registers and LDS): 2 layers, T = 4, B = 32."""
    cfg = li.custom_config(2, 4096, 4096, 32, 4, "bf16", cfg_id=820)
    inp = li.make_inputs(cfg)
    dy, dhT, dcT = upstream(cfg, 821)
    say("backward H=4096 L=2 T=4 B=32 bf16")
    run_and_check(inp, dy, dhT, dcT, dev, "bwd H4096")


# the on-chip recurrent chain (bf16 H = 4096, B <= 32): one column tile, a
# ragged second tile, and no upstream state gradients (dh0 / dc0 still out)
@pytest.mark.parametrize("B,states", [(16, True), (20, False), (32, False)])
def test_gpu_backward_on_chip_chain(dev, B, states):
    cfg = li.custom_config(1, 512, 4096, B, 5, "bf16", cfg_id=840 + B)
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 850 + B, with_states=states)
    say(f"backward on-chip chain H=4096 L=1 T=5 B={B} states={states}")
    run_and_check(inp, dy, dhT, dcT, dev, f"bwd chain H4096 B={B}")


# the on-chip chain at its other shapes: every (dtype, H) it is built for
# below H = 4096, one to four batch tiles (a third tile runs as a padded
# fourth), with and without upstream state gradients
ON_CHIP = [
    # L, I, H, B, T, dtype, states
    (2, 48, 128, 24, 5, "bf16", True),
    (2, 64, 256, 40, 5, "bf16", True),
    (1, 96, 512, 20, 6, "bf16", False),
    (1, 128, 1024, 5, 4, "bf16", True),
    (1, 64, 1536, 4, 5, "bf16", False),
    (1, 64, 2048, 64, 3, "bf16", True),
    (1, 64, 3072, 32, 3, "bf16", False),
    (1, 64, 128, 8, 6, "f32", False),
    (2, 48, 256, 33, 5, "f32", True),
    (1, 64, 512, 16, 4, "f32", False),
    (1, 32, 1024, 48, 3, "f32", True),
]


@pytest.mark.parametrize("shape", ON_CHIP, ids=[f"{s[5]}-H{s[2]}-B{s[3]}-L{s[0]}" for s in ON_CHIP])
def test_gpu_backward_on_chip_chain_shapes(dev, shape):
    import stacked_lstm_forward_amd as sl
    L, I, H, B, T, dtype, states = shape
    assert sl.lstm_bwd_chain_on_chip(sl.make_desc(L, I, H, B, T, dtype))
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=900 + H + B + L)
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 910 + H + B, with_states=states)
    say(f"backward on-chip chain {shape}")
    run_and_check(inp, dy, dhT, dcT, dev, f"bwd chain {dtype} H{H} B{B} L{L}")


def test_gpu_backward_wavefront_and_layerwise_forward_agree(dev):
    """The training forward saves the same activations in both schedules."""
    import stacked_lstm_forward_amd as sl
    cfg = li.custom_config(3, 64, 128, 16, 6, "bf16", cfg_id=830)
    d = sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype)
    assert sl.lstm_fwd_plan(d).as_dict()["regime"] == "wavefront"
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 831)
    say("backward after a wavefront forward")
    run_and_check(inp, dy, dhT, dcT, dev, "bwd wavefront L3 H128")


# dx, dh0 and dc0 are optional outputs (NULL: not written); the weight
# gradients must not depend on them: the on-chip chain (bf16 H = 4096 and 256,
# fp32 H = 512) and the streamed chain, with and without a dh0 iteration
@pytest.mark.parametrize("shape", [(1, 512, 4096, 16, 3, "bf16"), (2, 24, 20, 3, 5, "f32"), (2, 64, 64, 16, 4, "bf16"),
                                   (2, 64, 256, 24, 4, "bf16"), (1, 32, 512, 8, 3, "f32")])
def test_gpu_backward_without_input_gradients(dev, shape):
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    L, I, H, B, T, dtype = shape
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=870 + H + B)
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 880 + H)
    say(f"backward without dx/dh0/dc0 {shape}")
    tp = runner.prepare_train(inp, dy, dhT, dcT, dev)
    tp.dx = tp.dh0 = tp.dc0 = None
    tp.forward()
    tp.backward()
    assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_OK
    f32 = lambda a: None if a is None else np.asarray(a, dtype=np.float32).astype(np.float64)  # noqa: E731
    ref = orcb.lstm_backward_inputs(inp, f32(dy), f32(dhT), f32(dcT))
    dW = tp.dW.double().cpu().numpy()
    offs = [0, 4 * H * I] + [4 * H * I + k * 4 * H * H for k in range(1, L)]
    got_dW = [dW[offs[l]:offs[l] + 4 * H * (I if l == 0 else H)].reshape(4 * H, -1) for l in range(L)]
    got_dR = list(tp.dR.double().cpu().numpy().reshape(L, 4 * H, H))
    got_db = list(tp.db.double().cpu().numpy().reshape(L, 4 * H))
    tol = TOL[dtype]
    errs = {"dW": max(rel_err(g, r) for g, r in zip(got_dW, ref["dW"])),
            "dR": max(rel_err(g, r) for g, r in zip(got_dR, ref["dR"])),
            "db": max(rel_err(g, r) for g, r in zip(got_db, ref["db"]))}
    say(f"no dx/dh0/dc0 {shape}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    record(f"bwd no-input-grads {shape}", tol, errs)
    for k, v in errs.items():
        assert np.isfinite(v) and v <= tol, (shape, k, v)


def test_gpu_backward_plain_launch_options(dev):
    """lstm_fwd_train_ex / lstm_bwd_ex with plain (non-cooperative) launches
    give the same bits as the default entry points (the on-chip chain)."""
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    cfg = li.custom_config(1, 512, 4096, 20, 3, "bf16", cfg_id=890)
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 891)
    say("backward with plain-launch options")
    a = runner.prepare_train(inp, dy, dhT, dcT, dev)
    a.forward()
    a.backward()
    b = runner.prepare_train(inp, dy, dhT, dcT, dev)
    b.forward(plain_launch=True)
    b.backward(plain_launch=True)
    assert sl.lstm_bwd_last_error(b.bws) == sl.LSTM_OK
    for x, y in ((a.dx, b.dx), (a.dh0, b.dh0), (a.dc0, b.dc0), (a.dW, b.dW), (a.dR, b.dR), (a.db, b.db)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


# bitwise determinism of the on-chip chain's shapes (fixed summation orders:
# the K-group sums in LDS, the partial sums across workgroups, the K ranges of
# the gradient products): two backward passes on one workspace
@pytest.mark.parametrize("shape", [(2, 64, 256, 40, 5, "bf16"), (1, 64, 1536, 4, 6, "bf16"), (1, 32, 1024, 48, 3, "f32")],
                         ids=["bf16-H256-groups", "bf16-H1536-quarters", "f32-H1024-quarters-groups"])
def test_gpu_backward_bitwise_repeatable(dev, shape):
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    L, I, H, B, T, dtype = shape
    assert sl.lstm_bwd_chain_on_chip(sl.make_desc(L, I, H, B, T, dtype))
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=950 + H + B)
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 960 + H)
    say(f"backward repeatability {shape}")
    tp = runner.prepare_train(inp, dy, dhT, dcT, dev)
    tp.forward()
    tp.backward()
    first = [t.clone() for t in (tp.dx, tp.dh0, tp.dc0, tp.dW, tp.dR, tp.db)]
    for t in (tp.dx, tp.dh0, tp.dc0, tp.dW, tp.dR, tp.db):
        t.fill_(0)
    tp.backward()
    assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_OK
    for a, b in zip(first, (tp.dx, tp.dh0, tp.dc0, tp.dW, tp.dR, tp.db)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), shape


def test_gpu_backward_unaligned_upstream_gradient(dev):
    """dy not 16-byte aligned (a view 4 bytes into a buffer): the on-chip
    chain, which moves the per-step tensors 16 bytes at a time, is passed over
    for the streamed chain, and the gradients still match the oracle."""
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    cfg = li.custom_config(1, 64, 256, 16, 4, "bf16", cfg_id=990)
    assert sl.lstm_bwd_chain_on_chip(sl.make_desc(cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype))
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 991)
    say("backward with a misaligned dy")
    tp = runner.prepare_train(inp, dy, dhT, dcT, dev)
    buf = torch.empty(tp.dy.numel() + 1, dtype=torch.float32, device=dev)
    view = buf[1:].view_as(tp.dy)
    view.copy_(tp.dy)
    assert view.data_ptr() % 16 != 0
    tp.dy = view
    tp.forward()
    tp.backward()
    assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_OK
    got = tp.grads_f64()
    f32 = lambda a: None if a is None else np.asarray(a, dtype=np.float32).astype(np.float64)  # noqa: E731
    ref = orcb.lstm_backward_inputs(inp, f32(dy), f32(dhT), f32(dcT))
    errs = {k: rel_err(got[k], ref[k]) for k in ("dx", "dh0", "dc0")}
    for k in ("dW", "dR", "db"):
        errs[k] = max(rel_err(g, r) for g, r in zip(got[k], ref[k]))
    say("misaligned dy: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert np.isfinite(v) and v <= TOL["bf16"], (k, v)


@pytest.mark.parametrize("shape", [(1, 64, 256, 16, 4, "bf16"), (1, 64, 1024, 16, 3, "bf16")],
                         ids=["one-M-tile", "K-quarters"])
def test_gpu_backward_forced_wait_timeout(dev, shape):
    """A negative wait limit fails every blocked step wait of the on-chip chain
    at once: the kernel exits normally, lstm_bwd_last_error reports the
    timeout, and the next call on the same workspace is clean and correct."""
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    L, I, H, B, T, dtype = shape
    assert sl.lstm_bwd_chain_on_chip(sl.make_desc(L, I, H, B, T, dtype))
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=995 + H)
    inp = li.make_inputs(cfg, random_state=True)
    dy, dhT, dcT = upstream(cfg, 996)
    say(f"backward forced timeout {shape}")
    tp = runner.prepare_train(inp, dy, dhT, dcT, dev)
    tp.forward()
    o = sl.BwdOpts()
    o.wait_timeout_us = -1
    p = tp.fwd
    st = sl.lstm_bwd_ex(p.desc, p.x, p.h0, p.c0, p.W, p.R, tp.reserve, tp.dy, tp.dhT, tp.dcT, tp.dx, tp.dh0, tp.dc0,
                        tp.dW, tp.dR, tp.db, tp.bws, None, o)
    assert st == sl.LSTM_OK
    assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_ERR_BARRIER_TIMEOUT
    tp.backward()  # the same workspace and buffers, default limit
    assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_OK
    got = tp.grads_f64()
    f32 = lambda a: None if a is None else np.asarray(a, dtype=np.float32).astype(np.float64)  # noqa: E731
    ref = orcb.lstm_backward_inputs(inp, f32(dy), f32(dhT), f32(dcT))
    errs = {k: rel_err(got[k], ref[k]) for k in ("dx", "dh0", "dc0")}
    for k in ("dW", "dR", "db"):
        errs[k] = max(rel_err(g, r) for g, r in zip(got[k], ref[k]))
    say(f"after forced timeout {shape}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert np.isfinite(v) and v <= TOL[dtype], (k, v)
