"""lstm_fwd_noalloc (the forward pass with the library's fixed device scratch
instead of a caller's workspace) against lstm_fwd on the same inputs, through
the C ABI: two calls in a row, the second on a smaller problem, each bit for bit
equal to lstm_fwd and within the dtype's tolerance of the fp64 oracle.
"""
import numpy as np
import pytest

import lstm_inputs as li
import oracle.lstm_oracle as orc
from tests.pins import rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run_both(inp):
    import torch
    import stacked_lstm_forward_amd as sl
    from stacked_lstm_forward_amd import runner
    ref = runner.prepare(inp, "cuda:0")
    ref.run()
    assert sl.lstm_fwd_last_error(ref.ws) == sl.LSTM_OK
    p = runner.prepare(inp, "cuda:0")
    for t in (p.y, p.hT) + ((p.cT,) if p.cT is not None else ()):
        t.fill_(7)  # outputs must be written, not left over
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    st = sl.lstm_fwd_noalloc(p.desc, p.x, p.h0, p.c0, p.W, p.R, p.b, p.y, p.hT, p.cT, status)
    assert st == sl.LSTM_OK, sl.lstm_status_string(st)
    torch.cuda.synchronize()
    assert int(status.item()) == sl.LSTM_OK
    for a, b in zip((ref.y, ref.hT, ref.cT), (p.y, p.hT, p.cT)):
        if a is None:
            assert b is None
            continue
        assert torch.equal(_bits(a), _bits(b))
    return p.outputs_f32()


def test_noalloc_matches_workspace_call_twice_second_smaller():
    import torch
    import stacked_lstm_forward_amd as sl
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sl.load_library()
    cases = [li.custom_config(2, 256, 256, 16, 24, "bf16", cfg_id=701),
             li.custom_config(1, 64, 128, 4, 8, "f32", cfg_id=702)]
    sizes = [sl.lstm_fwd_workspace_size(sl.make_desc(c.L, c.I, c.H, c.B, c.T, c.dtype)) for c in cases]
    assert sizes[0] > sizes[1] and sizes[0] <= sl.NOALLOC_MAX_WORKSPACE
    for cfg in cases:
        say(f"noalloc {cfg.name}")
        inp = li.make_inputs(cfg, random_state=True)
        got = _run_both(inp)
        ref = orc.lstm_forward_inputs(inp)
        for n, g, r in zip(("y", "hT", "cT"), got, ref):
            e = rel_err(g, r)
            say(f"  {n}={e:.2e}")
            assert np.all(np.isfinite(g)) and e <= TOL[cfg.dtype], (cfg.name, n, e)


def test_noalloc_refuses_problems_beyond_its_scratch():
    import stacked_lstm_forward_amd as sl
    sl.load_library()
    c = li.CONFIGS["c2"]  # needs 113 MiB of workspace
    d = sl.make_desc(c.L, c.I, c.H, c.B, c.T, c.dtype)
    assert sl.lstm_fwd_workspace_size(d) > sl.NOALLOC_MAX_WORKSPACE
    fake = 1 << 20
    st = sl.lstm_fwd_noalloc(d, fake, None, None, fake, fake, fake, fake, None, None, None, 0)
    assert st == sl.LSTM_ERR_WORKSPACE
