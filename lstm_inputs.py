"""Seeded synthetic inputs for the stacked recurrent forward pass (LSTM, GRU, simple RNN).

This module holds shapes, seeds, value distributions and storage formats only.
It contains none of the LSTM arithmetic: both the fp64 CPU oracle (``oracle/``)
and the HIP path (``stacked_lstm_forward_amd``) consume what it produces, and it
imports neither of them.

Workloads (the five stacked-LSTM shapes that the pages' large-hidden /
small-batch / small-deep regimes call for; "Optimizing Performance of Recurrent
Neural Networks on GPUs", key results on layer overlap at hidden 4096 and the
minibatch-32 question; "Persistent RNNs" on small batches):

    c1  L=1  I=H=128   B=8   T=16    fp32
    c2  L=4  I=H=512   B=64  T=100   fp32
    c3  L=8  I=H=256   B=64  T=200   bf16 weights/x, fp32 cell state
    c4  L=4  I=H=4096  B=32  T=50    bf16 weights/x, fp32 cell state
    c5  L=1  I=H=1536  B=4   T=2048  bf16 weights/x, fp32 cell state

Distributions: W, R, b ~ U(-1/sqrt(H), 1/sqrt(H)); x ~ N(0, 1); h0 = c0 = 0
unless a test asks for random initial states.  Gate blocks inside W, R, b are
ordered i, f, g, o (LSTM); r, z, n with bias blocks b_r, b_z, b_Wn, b_Rn
(GRU); a simple RNN has one block.  Row counts per cell are in ``ROWS``.

Seeds: ``np.random.default_rng([cfg_id, layer, tensor_id])`` with tensor_id
W=0, R=1, b=2; x uses ``[cfg_id, 1000, 0]``; random h0/c0 use
``[cfg_id, 2000 + layer, 3 or 4]``.

bf16 values are generated in fp64, rounded to fp32 (round-to-nearest-even) and
then to bf16 (round-to-nearest-even on the fp32 bits).  Both sides see exactly
those bf16 values: the GPU receives the raw bits, the oracle receives them
widened exactly (bf16 -> fp32 -> fp64 are exact widenings).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

DTYPES = ("f32", "bf16")
CELLS = ("lstm", "gru", "rnn_tanh", "rnn_relu")
# (weight-row blocks, bias blocks) per cell, in multiples of H
ROWS = {"lstm": (4, 4), "gru": (3, 4), "rnn_tanh": (1, 1), "rnn_relu": (1, 1)}


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    L: int
    I: int
    H: int
    B: int
    T: int
    dtype: str
    cell: str = "lstm"

    @property
    def gates(self) -> int:
        return ROWS[self.cell][0]

    @property
    def flops(self) -> int:
        """2 * G*H * (I_l + H) * B * T summed over layers, G = 4 (LSTM), 3 (GRU), 1 (RNN);
        bias and pointwise work excluded."""
        tot = 0
        for l in range(self.L):
            il = self.I if l == 0 else self.H
            tot += 2 * self.gates * self.H * (il + self.H) * self.B * self.T
        return tot


CONFIGS: Dict[str, Config] = {
    "c1": Config("c1", 1, L=1, I=128, H=128, B=8, T=16, dtype="f32"),
    "c2": Config("c2", 2, L=4, I=512, H=512, B=64, T=100, dtype="f32"),
    "c3": Config("c3", 3, L=8, I=256, H=256, B=64, T=200, dtype="bf16"),
    "c4": Config("c4", 4, L=4, I=4096, H=4096, B=32, T=50, dtype="bf16"),
    "c5": Config("c5", 5, L=1, I=1536, H=1536, B=4, T=2048, dtype="bf16"),
}


def custom_config(L: int, I: int, H: int, B: int, T: int, dtype: str, cfg_id: int = 99,
                  cell: str = "lstm") -> Config:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}")
    if cell not in CELLS:
        raise ValueError(f"cell must be one of {CELLS}")
    tag = "" if cell == "lstm" else cell
    return Config(f"{tag}L{L}I{I}H{H}B{B}T{T}{dtype}", cfg_id, L, I, H, B, T, dtype, cell)


def with_cell(cfg: Config, cell: str) -> Config:
    """The same shapes and seeds with another cell."""
    return Config(f"{cfg.name}-{cell}", cfg.cfg_id, cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype, cell)


# ----------------------------------------------------------------------------- formats
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even), returning the raw uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to fp32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values -> storage array (float32, or uint16 bf16 bits)."""
    a32 = np.asarray(a64, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(a32)
    if dtype == "bf16":
        return bf16_bits_from_f32(a32)
    raise ValueError(dtype)


def exact_f32(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> the exact values it holds, as float32 (exact for both dtypes)."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32)
    return f32_from_bf16_bits(stored)


# ----------------------------------------------------------------------------- inputs
@dataclass
class Inputs:
    """Storage-form tensors of one workload.

    x: [T, B, I]; W[l]: [G*H, I_l]; R[l]: [G*H, H]; b[l]: [NB*H] with (G, NB) = ROWS[cell];
    h0: [L, B, H] (dtype); c0: [L, B, H] (always fp32, LSTM only).  Storage is float32 for "f32" and uint16 bf16 bits
    for "bf16".  h0 / c0 are None for zero initial states.
    """

    cfg: Config
    x: np.ndarray
    W: List[np.ndarray]
    R: List[np.ndarray]
    b: List[np.ndarray]
    h0: Optional[np.ndarray] = None
    c0: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    # exact values as float32 (the oracle widens these to fp64)
    def x_f32(self) -> np.ndarray:
        return exact_f32(self.x, self.cfg.dtype)

    def W_f32(self, l: int) -> np.ndarray:
        return exact_f32(self.W[l], self.cfg.dtype)

    def R_f32(self, l: int) -> np.ndarray:
        return exact_f32(self.R[l], self.cfg.dtype)

    def b_f32(self, l: int) -> np.ndarray:
        return exact_f32(self.b[l], self.cfg.dtype)

    def h0_f32(self) -> Optional[np.ndarray]:
        return None if self.h0 is None else exact_f32(self.h0, self.cfg.dtype)

    def c0_f32(self) -> Optional[np.ndarray]:
        return None if self.c0 is None else np.asarray(self.c0, dtype=np.float32)

    # packed C-ABI layout
    def packed(self) -> Dict[str, Optional[np.ndarray]]:
        """Contiguous arrays in the library's layout: W = W_0 ++ W_1 ++ ..., R = [L,G*H,H], b = [L,NB*H]."""
        return {
            "x": np.ascontiguousarray(self.x),
            "W": np.concatenate([w.reshape(-1) for w in self.W]),
            "R": np.ascontiguousarray(np.stack(self.R)),
            "b": np.ascontiguousarray(np.stack(self.b)),
            "h0": None if self.h0 is None else np.ascontiguousarray(self.h0),
            "c0": None if self.c0 is None else np.ascontiguousarray(self.c0, dtype=np.float32),
        }

    def batch_subset(self, idx) -> "Inputs":
        """The same workload restricted to batch columns ``idx`` (sequences are independent)."""
        idx = np.asarray(idx)
        cfg = Config(self.cfg.name + "-sub", self.cfg.cfg_id, self.cfg.L, self.cfg.I, self.cfg.H,
                     len(idx), self.cfg.T, self.cfg.dtype, self.cfg.cell)
        return Inputs(cfg, np.ascontiguousarray(self.x[:, idx]), self.W, self.R, self.b,
                      None if self.h0 is None else np.ascontiguousarray(self.h0[:, idx]),
                      None if self.c0 is None else np.ascontiguousarray(self.c0[:, idx]),
                      dict(self.meta, batch_subset=idx.tolist()))


def _uniform(rng: np.random.Generator, shape, bound: float) -> np.ndarray:
    return rng.uniform(-bound, bound, size=shape)


def make_inputs(cfg: Config, random_state: bool = False, state_scale: float = 0.5) -> Inputs:
    """Generate the seeded synthetic workload ``cfg``.

    random_state=False gives h0 = c0 = None (zero initial states, the workloads'
    definition); True draws h0, c0 ~ U(-state_scale, state_scale) for tests.
    """
    L, I, H, B, T, dt = cfg.L, cfg.I, cfg.H, cfg.B, cfg.T, cfg.dtype
    G, NB = ROWS[cfg.cell]
    bound = 1.0 / np.sqrt(H)
    W, R, b = [], [], []
    for l in range(L):
        il = I if l == 0 else H
        W.append(to_storage(_uniform(np.random.default_rng([cfg.cfg_id, l, 0]), (G * H, il), bound), dt))
        R.append(to_storage(_uniform(np.random.default_rng([cfg.cfg_id, l, 1]), (G * H, H), bound), dt))
        b.append(to_storage(_uniform(np.random.default_rng([cfg.cfg_id, l, 2]), (NB * H,), bound), dt))
    x = to_storage(np.random.default_rng([cfg.cfg_id, 1000, 0]).standard_normal((T, B, I)), dt)
    h0 = c0 = None
    if random_state:
        h0 = np.stack([to_storage(_uniform(np.random.default_rng([cfg.cfg_id, 2000 + l, 3]), (B, H), state_scale), dt)
                       for l in range(L)])
        c0 = np.stack([_uniform(np.random.default_rng([cfg.cfg_id, 2000 + l, 4]), (B, H), state_scale).astype(np.float32)
                       for l in range(L)])
    meta = {"seed_scheme": "default_rng([cfg_id, layer, tensor_id]); W=0 R=1 b=2; x=[cfg_id,1000,0]; "
                           "h0/c0=[cfg_id,2000+layer,3|4]",
            "cfg_id": cfg.cfg_id, "random_state": random_state}
    return Inputs(cfg, x, W, R, b, h0, c0, meta)


def from_arrays(L: int, I: int, H: int, B: int, T: int, dtype: str, x64, W64, R64, b64,
                h064=None, c064=None, cell: str = "lstm") -> Inputs:
    """Build storage-form inputs from explicit fp64 arrays (structured pin inputs)."""
    cfg = custom_config(L, I, H, B, T, dtype, cell=cell)
    G, NB = ROWS[cell]
    x = to_storage(np.asarray(x64, dtype=np.float64).reshape(T, B, I), dtype)
    W = [to_storage(np.asarray(W64[l], dtype=np.float64).reshape(G * H, I if l == 0 else H), dtype) for l in range(L)]
    R = [to_storage(np.asarray(R64[l], dtype=np.float64).reshape(G * H, H), dtype) for l in range(L)]
    b = [to_storage(np.asarray(b64[l], dtype=np.float64).reshape(NB * H), dtype) for l in range(L)]
    h0 = None if h064 is None else to_storage(np.asarray(h064, dtype=np.float64).reshape(L, B, H), dtype)
    c0 = None if c064 is None else np.asarray(c064, dtype=np.float64).reshape(L, B, H).astype(np.float32)
    return Inputs(cfg, x, W, R, b, h0, c0, {"structured": True})
