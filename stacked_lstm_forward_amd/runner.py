"""Torch plumbing around the C ABI: device copies of host arrays, output and
workspace allocation, and one call of ``lstm_fwd``.  No cell arithmetic here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import (LSTM_BF16, LSTM_F32, BwdOpts, LstmDesc, LstmOpts, check, lstm_bwd, lstm_bwd_ex,
               lstm_bwd_workspace_size, lstm_fwd, lstm_fwd_ex, lstm_fwd_train, lstm_fwd_train_ex,
               lstm_fwd_workspace_size, lstm_train_reserve_size, make_desc)


def _torch():
    import torch
    return torch


def to_device_array(a: Optional[np.ndarray], dtype: str, device):
    """Storage array (float32, or uint16 bf16 bits) -> device tensor (float32 / bfloat16)."""
    torch = _torch()
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    return t.to(device)


@dataclass
class DeviceProblem:
    desc: LstmDesc
    x: object
    W: object
    R: object
    b: object
    h0: object
    c0: object
    y: object
    hT: object
    cT: object
    ws: object
    ws_bytes: int

    def run(self, stream=None, opts: Optional[LstmOpts] = None) -> None:
        if opts is None:
            st = lstm_fwd(self.desc, self.x, self.h0, self.c0, self.W, self.R, self.b, self.y, self.hT, self.cT,
                          self.ws, stream)
        else:
            st = lstm_fwd_ex(self.desc, self.x, self.h0, self.c0, self.W, self.R, self.b, self.y, self.hT,
                             self.cT, self.ws, stream, opts)
        check(st, "lstm_fwd")

    def outputs_f32(self):
        """(y, hT, cT) as float32 numpy arrays (synchronises); cT is None for cells without one."""
        return (self.y.float().cpu().numpy(), self.hT.float().cpu().numpy(),
                None if self.cT is None else self.cT.float().cpu().numpy())


def workspace(desc: LstmDesc, device):
    """A 256-byte aligned uint8 workspace tensor of lstm_fwd_workspace_size(desc) bytes."""
    torch = _torch()
    n = lstm_fwd_workspace_size(desc)
    if n == 0:
        raise ValueError("unsupported problem: lstm_fwd_workspace_size returned 0")
    raw = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + n], n


def prepare(inp, device="cuda:0") -> DeviceProblem:
    """Copy an ``lstm_inputs.Inputs`` to the device and allocate outputs and workspace."""
    torch = _torch()
    c = inp.cfg
    cell = getattr(c, "cell", "lstm")
    desc = make_desc(c.L, c.I, c.H, c.B, c.T, c.dtype, cell)
    pk = inp.packed()
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    x = to_device_array(pk["x"], c.dtype, device)
    W = to_device_array(pk["W"], c.dtype, device)
    R = to_device_array(pk["R"], c.dtype, device)
    b = to_device_array(pk["b"], c.dtype, device)
    h0 = to_device_array(pk["h0"], c.dtype, device)
    c0 = None if pk["c0"] is None else torch.from_numpy(pk["c0"]).to(device)
    y = torch.empty((c.T, c.B, c.H), dtype=tdt, device=device)
    hT = torch.empty((c.L, c.B, c.H), dtype=tdt, device=device)
    cT = torch.empty((c.L, c.B, c.H), dtype=torch.float32, device=device) if cell == "lstm" else None
    ws, n = workspace(desc, device)
    return DeviceProblem(desc, x, W, R, b, h0, c0, y, hT, cT, ws, n)


def forward(inp, device="cuda:0", opts: Optional[LstmOpts] = None):
    """Run the HIP forward pass on ``inp``; returns float32 numpy (y, hT, cT)."""
    prob = prepare(inp, device)
    prob.run(opts=opts)
    return prob.outputs_f32()




@dataclass
class TrainProblem:
    """A DeviceProblem plus what one training forward and one backward call need:
    the reserve buffer, the backward workspace, the upstream gradients and the
    gradient outputs (all fp32)."""
    fwd: DeviceProblem
    reserve: object
    bws: object
    dy: object
    dhT: object
    dcT: object
    dx: object
    dh0: object
    dc0: object
    dW: object
    dR: object
    db: object

    def forward(self, stream=None, plain_launch=False) -> None:
        p = self.fwd
        if plain_launch:
            o = LstmOpts()
            o.plain_launch = 1
            check(lstm_fwd_train_ex(p.desc, p.x, p.h0, p.c0, p.W, p.R, p.b, p.y, p.hT, p.cT, self.reserve, p.ws,
                                    stream, o), "lstm_fwd_train_ex")
            return
        check(lstm_fwd_train(p.desc, p.x, p.h0, p.c0, p.W, p.R, p.b, p.y, p.hT, p.cT, self.reserve, p.ws, stream),
              "lstm_fwd_train")

    def backward(self, stream=None, plain_launch=False) -> None:
        p = self.fwd
        if plain_launch:
            o = BwdOpts()
            o.plain_launch = 1
            check(lstm_bwd_ex(p.desc, p.x, p.h0, p.c0, p.W, p.R, self.reserve, self.dy, self.dhT, self.dcT, self.dx,
                              self.dh0, self.dc0, self.dW, self.dR, self.db, self.bws, stream, o), "lstm_bwd_ex")
            return
        check(lstm_bwd(p.desc, p.x, p.h0, p.c0, p.W, p.R, self.reserve, self.dy, self.dhT, self.dcT, self.dx,
                       self.dh0, self.dc0, self.dW, self.dR, self.db, self.bws, stream), "lstm_bwd")

    def grads_f64(self):
        """Gradients as float64 numpy arrays, split per layer like the oracle's (synchronises)."""
        c = self.fwd.desc
        L, I, H = c.L, c.I, c.H
        dW = self.dW.double().cpu().numpy()
        offs = [0, 4 * H * I] + [4 * H * I + k * 4 * H * H for k in range(1, L)]
        return {"dx": self.dx.double().cpu().numpy(), "dh0": self.dh0.double().cpu().numpy(),
                "dc0": self.dc0.double().cpu().numpy(),
                "dW": [dW[offs[l]:offs[l] + 4 * H * (I if l == 0 else H)].reshape(4 * H, -1) for l in range(L)],
                "dR": list(self.dR.double().cpu().numpy().reshape(L, 4 * H, H)),
                "db": list(self.db.double().cpu().numpy().reshape(L, 4 * H))}


def aligned_buffer(nbytes: int, device):
    torch = _torch()
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + nbytes]


def prepare_train(inp, dy, dhT=None, dcT=None, device="cuda:0") -> TrainProblem:
    """Device buffers for lstm_fwd_train + lstm_bwd on an LSTM ``lstm_inputs.Inputs``;
    dy [T, B, H] and dhT / dcT [L, B, H] (or None) are host arrays of upstream gradients."""
    torch = _torch()
    p = prepare(inp, device)
    c = inp.cfg
    rs = lstm_train_reserve_size(p.desc)
    wb = lstm_bwd_workspace_size(p.desc)
    if rs == 0 or wb == 0:
        raise ValueError("training passes need an LSTM problem the library supports")
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)  # noqa: E731
    nW = 4 * c.H * c.I + (c.L - 1) * 4 * c.H * c.H
    z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=device)  # noqa: E731
    return TrainProblem(p, aligned_buffer(rs, device), aligned_buffer(wb, device), f32(dy), f32(dhT), f32(dcT),
                        z(c.T, c.B, c.I), z(c.L, c.B, c.H), z(c.L, c.B, c.H), z(nW), z(c.L, 4 * c.H, c.H),
                        z(c.L, 4 * c.H))


__all__ = ["DeviceProblem", "TrainProblem", "prepare", "prepare_train", "forward", "workspace", "aligned_buffer",
           "to_device_array", "LSTM_F32", "LSTM_BF16"]
