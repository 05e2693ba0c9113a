"""GPU: the forward pass, and a whole training step (forward keeping state and
backward), captured in a HIP graph (stream capture through torch.cuda.graph)
and replayed.  Every replay must reproduce the eager call's
outputs bit for bit, with eager work (clearing the outputs) and
synchronisations between the replays.  Persistent kernels are captured with
plain launches (lstm_fwd_opts_t.plain_launch); the step counters are cleared by
kernels inside the captured work (no memset node), so every replay starts
from zero.  Every case prints its name before touching the GPU.
"""
import pytest

import lstm_inputs as li

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import stacked_lstm_forward_amd as sl
    sl.load_library()
    return "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    # name, (L, I, H, B, T, dtype), random initial states
    ("layerwise fp32 (one small layer)", (1, 128, 128, 8, 16, "f32"), False),
    ("wavefront bf16 (three layers)", (3, 64, 64, 16, 6, "bf16"), True),
    ("register-resident bf16 H=4096", (1, 256, 4096, 16, 3, "bf16"), True),
]


@pytest.mark.parametrize("name,shape,rs", CASES, ids=[c[0] for c in CASES])
def test_gpu_graph_replay(dev, name, shape, rs):
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    L, I, H, B, T, dtype = shape
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=900 + H + L)
    inp = li.make_inputs(cfg, random_state=rs)
    say(f"graph replay: {name}")
    prob = runner.prepare(inp, dev)
    opts = sl.LstmOpts()
    opts.plain_launch = 1
    prob.run(opts=opts)  # eager; also sets the kernels' attributes before the capture
    assert sl.lstm_fwd_last_error(prob.ws) == sl.LSTM_OK
    outs = [t for t in (prob.y, prob.hT, prob.cT) if t is not None]
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        prob.run(stream=s, opts=opts)
    torch.cuda.synchronize()
    for k in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert sl.lstm_fwd_last_error(prob.ws) == sl.LSTM_OK, (name, k)
        for a, b in zip(ref, outs):
            assert torch.equal(bits(a), bits(b)), (name, k)


TRAIN_CASES = [
    # name, (L, I, H, B, T, dtype)
    ("training step, chain over all of K (bf16 H=256)", (2, 64, 256, 32, 5, "bf16")),
    ("training step, chain over K quarters (fp32 H=1024)", (1, 32, 1024, 16, 3, "f32")),
]


@pytest.mark.parametrize("name,shape", TRAIN_CASES, ids=[c[0] for c in TRAIN_CASES])
def test_gpu_graph_replay_training(dev, name, shape):
    """lstm_fwd_train + lstm_bwd with plain launches captured together in one
    graph: every replay reproduces the eager gradients bit for bit."""
    import numpy as np
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    L, I, H, B, T, dtype = shape
    assert sl.lstm_bwd_chain_on_chip(sl.make_desc(L, I, H, B, T, dtype))
    cfg = li.custom_config(L, I, H, B, T, dtype, cfg_id=970 + H + L)
    inp = li.make_inputs(cfg, random_state=True)
    rng = np.random.default_rng(971)
    dy = rng.standard_normal((T, B, H))
    dhT = rng.standard_normal((L, B, H))
    dcT = rng.standard_normal((L, B, H))
    say(f"graph replay: {name}")
    tp = runner.prepare_train(inp, dy, dhT, dcT, dev)
    tp.forward(plain_launch=True)  # eager; also sets the kernels' attributes before the capture
    tp.backward(plain_launch=True)
    assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_OK
    outs = [tp.dx, tp.dh0, tp.dc0, tp.dW, tp.dR, tp.db]
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tp.forward(stream=s, plain_launch=True)
        tp.backward(stream=s, plain_launch=True)
    torch.cuda.synchronize()
    for k in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert sl.lstm_bwd_last_error(tp.bws) == sl.LSTM_OK, (name, k)
        for a, b in zip(ref, outs):
            assert torch.equal(bits(a), bits(b)), (name, k)
