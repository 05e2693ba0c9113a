"""Plain fp64 CPU oracle of the stacked recurrent forward pass (LSTM, GRU, plain RNN).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It is
slow on purpose: per layer, per timestep, one library matrix product for each of
the two weight products, then the gate non-linearities elementwise.  Nothing is
blocked, fused or reordered beyond what the definition below states.

What is computed (the standard forget-gate LSTM that the cuDNN-v5 work in
"Optimizing Performance of Recurrent Neural Networks on GPUs" optimises; its
"proposed method" section groups the four per-gate matrices into one 4H-row
matrix and keeps the input-weight and recurrent-weight products as two
independent products; its layer-overlap item stacks layers so that layer l's
output sequence is layer l+1's input):

    for each layer l, with u_t = x_t (l = 0) or h^{l-1}_t (l >= 1):
        p   = W_l u_t + R_l h_{t-1} + b_l          (4H rows, gate blocks i, f, g, o)
        i   = sigma(p[0:H]),  f = sigma(p[H:2H]),  g = tanh(p[2H:3H]),  o = sigma(p[3H:4H])
        c_t = f * c_{t-1} + i * g
        h_t = o * tanh(c_t)

Readings where the pages are silent (they print no equations, layouts or
examples): one bias vector per layer; gate order i, f, g, o; I_l = H for
l >= 1; time-major tensors x [T, B, I], y [T, B, H], states [L, B, H]; y holds
the top layer's h_1..h_T; missing h0 / c0 are zeros.  All arithmetic is fp64.

The same page applies its optimisations to GRU cells (three grouped
matrices) and to the simple RNN (one matrix per input, so nothing to group)
("Optimizing Performance of Recurrent Neural Networks on GPUs", proposed
method, last item); the pages print neither cell's equations.  Read as the
cuDNN-v5 cells that page measures against:

    GRU (gate blocks r, z, n of W_l [3H, I_l] and R_l [3H, H]; b_l [4H] holds
    b_r, b_z, b_Wn, b_Rn -- the r and z biases of the two products summed, the
    n gate's two biases kept apart because r multiplies only the recurrent one):
        r   = sigma(W_r u + R_r h + b_r)
        z   = sigma(W_z u + R_z h + b_z)
        n   = tanh(W_n u + b_Wn + r * (R_n h + b_Rn))
        h_t = (1 - z) * n + z * h_{t-1}
    simple RNN (W_l [H, I_l], R_l [H, H], b_l [H]):
        h_t = tanh(W u + R h + b)      ("rnn_tanh")
        h_t = max(0, W u + R h + b)    ("rnn_relu")

Neither has a cell state: cT is not produced (None).

Parity status: every function here is pinned by the CPU tests (closed forms for
H = 1 and for zero x / zero R, exact saturation, brute-force recursion in
40-digit arithmetic, torch.nn.LSTM / GRU / RNN in float64, layer / time /
batch invariants).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^{-z}) in fp64, evaluated without overflow.

    For z >= 0 it uses 1 / (1 + e^{-z}); for z < 0 it uses e^{z} / (1 + e^{z}).
    Both saturate to exactly 1.0 and 0.0 for large |z| (e.g. |z| >= 1e4).
    """
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    e = np.exp(z[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def lstm_cell(W: np.ndarray, R: np.ndarray, b: np.ndarray, u: np.ndarray, h: np.ndarray,
              c: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """One LSTM step for a batch (the single-cell level of the optimised network).

    W: [4H, I_l], R: [4H, H], b: [4H], u: [B, I_l], h, c: [B, H]  (all fp64).
    The four gate pre-activations come out of one grouped 4H-row product per
    weight matrix ("Optimizing Performance of Recurrent Neural Networks on
    GPUs", proposed method, gate grouping).  Returns (h', c').
    """
    H = R.shape[1]
    p = u @ W.T + h @ R.T + b          # [B, 4H]
    i = sigmoid(p[:, 0 * H:1 * H])
    f = sigmoid(p[:, 1 * H:2 * H])
    g = np.tanh(p[:, 2 * H:3 * H])
    o = sigmoid(p[:, 3 * H:4 * H])
    c_new = f * c + i * g
    h_new = o * np.tanh(c_new)
    return h_new, c_new


def gru_cell(W: np.ndarray, R: np.ndarray, b: np.ndarray, u: np.ndarray,
             h: np.ndarray) -> np.ndarray:
    """One GRU step for a batch (the cuDNN-v5 GRU; see the module docstring).

    W: [3H, I_l], R: [3H, H] with gate blocks r, z, n; b: [4H] = b_r, b_z, b_Wn, b_Rn;
    u: [B, I_l], h: [B, H].  One grouped product per weight matrix (three
    matrix groups).  Returns h'.
    """
    H = R.shape[1]
    xu = u @ W.T                       # [B, 3H]
    rh = h @ R.T                       # [B, 3H]
    r = sigmoid(xu[:, 0:H] + rh[:, 0:H] + b[0:H])
    z = sigmoid(xu[:, H:2 * H] + rh[:, H:2 * H] + b[H:2 * H])
    n = np.tanh(xu[:, 2 * H:3 * H] + b[2 * H:3 * H] + r * (rh[:, 2 * H:3 * H] + b[3 * H:4 * H]))
    return (1.0 - z) * n + z * h


def rnn_cell(W: np.ndarray, R: np.ndarray, b: np.ndarray, u: np.ndarray, h: np.ndarray,
             relu: bool) -> np.ndarray:
    """One simple-RNN step: act(W u + R h + b), act = tanh or max(0, .).

    W: [H, I_l], R: [H, H], b: [H]; u: [B, I_l], h: [B, H].  Returns h'.
    """
    p = u @ W.T + h @ R.T + b
    return np.maximum(p, 0.0) if relu else np.tanh(p)


CELLS = ("lstm", "gru", "rnn_tanh", "rnn_relu")
GATES = {"lstm": 4, "gru": 3, "rnn_tanh": 1, "rnn_relu": 1}   # row blocks of W_l and R_l
BIAS_ROWS = {"lstm": 4, "gru": 4, "rnn_tanh": 1, "rnn_relu": 1}  # multiples of H in b_l


def cell_layer(cell: str, W: np.ndarray, R: np.ndarray, b: np.ndarray, U: np.ndarray, h0: np.ndarray,
               c0: Optional[np.ndarray]) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """One layer of any cell over the whole sequence U: [T, B, I_l]; returns (Y, hT, cT or None)."""
    if cell == "lstm":
        return lstm_layer(W, R, b, U, h0, c0)
    T = U.shape[0]
    B, H = h0.shape
    Y = np.empty((T, B, H), dtype=np.float64)
    h = h0
    for t in range(T):
        h = gru_cell(W, R, b, U[t], h) if cell == "gru" else rnn_cell(W, R, b, U[t], h, cell == "rnn_relu")
        Y[t] = h
    return Y, h, None


def lstm_layer(W: np.ndarray, R: np.ndarray, b: np.ndarray, U: np.ndarray, h0: np.ndarray,
               c0: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Run one layer over the whole sequence U: [T, B, I_l].

    The recurrence is strictly serial in t; every unit is updated from the
    previous step's h (synchronous update).  Returns (Y [T, B, H], hT, cT).
    """
    T = U.shape[0]
    B, H = h0.shape
    Y = np.empty((T, B, H), dtype=np.float64)
    h, c = h0, c0
    for t in range(T):
        h, c = lstm_cell(W, R, b, U[t], h, c)
        Y[t] = h
    return Y, h, c


def lstm_forward(x: np.ndarray, W: Sequence[np.ndarray], R: Sequence[np.ndarray],
                 b: Sequence[np.ndarray], h0: Optional[np.ndarray] = None,
                 c0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Stacked LSTM forward pass in fp64 (the network level: layer l feeds layer l+1).

    x: [T, B, I]; W[l]: [4H, I_l]; R[l]: [4H, H]; b[l]: [4H]; h0, c0: [L, B, H] or None (zeros).
    Inputs of any float dtype are widened to fp64 layer by layer.
    Returns y [T, B, H] (top layer's h_1..h_T), hT [L, B, H], cT [L, B, H], all fp64.
    """
    L = len(W)
    U = np.asarray(x, dtype=np.float64)
    T, B, _ = U.shape
    H = np.asarray(R[0]).shape[1]
    hT = np.empty((L, B, H), dtype=np.float64)
    cT = np.empty((L, B, H), dtype=np.float64)
    for l in range(L):
        Wl = np.asarray(W[l], dtype=np.float64)
        Rl = np.asarray(R[l], dtype=np.float64)
        bl = np.asarray(b[l], dtype=np.float64)
        hl = np.zeros((B, H)) if h0 is None else np.asarray(h0[l], dtype=np.float64)
        cl = np.zeros((B, H)) if c0 is None else np.asarray(c0[l], dtype=np.float64)
        U, hT[l], cT[l] = lstm_layer(Wl, Rl, bl, U, hl, cl)
        del Wl, Rl
    return U, hT, cT


def rnn_forward(cell: str, x: np.ndarray, W: Sequence[np.ndarray], R: Sequence[np.ndarray],
                b: Sequence[np.ndarray], h0: Optional[np.ndarray] = None,
                c0: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Stacked forward pass of any cell in fp64 (layer l's output sequence feeds layer l+1).

    Shapes as lstm_forward with GATES[cell]*H weight rows and BIAS_ROWS[cell]*H
    biases; c0 is used by the LSTM only.  Returns y, hT and cT (None unless LSTM).
    """
    if cell not in CELLS:
        raise ValueError(cell)
    if cell == "lstm":
        return lstm_forward(x, W, R, b, h0, c0)
    L = len(W)
    U = np.asarray(x, dtype=np.float64)
    T, B, _ = U.shape
    H = np.asarray(R[0]).shape[1]
    hT = np.empty((L, B, H), dtype=np.float64)
    for l in range(L):
        hl = np.zeros((B, H)) if h0 is None else np.asarray(h0[l], dtype=np.float64)
        U, hT[l], _ = cell_layer(cell, np.asarray(W[l], dtype=np.float64), np.asarray(R[l], dtype=np.float64),
                                 np.asarray(b[l], dtype=np.float64), U, hl, None)
    return U, hT, None


def forward_inputs(inp) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Oracle on an ``lstm_inputs.Inputs`` object of any cell (exact stored values, widened to fp64)."""
    L = inp.cfg.L
    return rnn_forward(inp.cfg.cell, inp.x_f32(),
                       _LazyList(inp.W_f32, L), _LazyList(inp.R_f32, L), _LazyList(inp.b_f32, L),
                       inp.h0_f32(), inp.c0_f32())


def lstm_forward_inputs(inp) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Oracle on an LSTM ``lstm_inputs.Inputs`` object (exact stored values, widened to fp64)."""
    if inp.cfg.cell != "lstm":
        raise ValueError("lstm_forward_inputs on a " + inp.cfg.cell + " workload; use forward_inputs")
    return forward_inputs(inp)


class _LazyList:
    """Sequence that materialises element l on access (keeps one layer's fp64 weights alive)."""

    def __init__(self, fn, n: int):
        self._fn, self._n = fn, n

    def __len__(self) -> int:
        return self._n

    def __getitem__(self, l: int):
        if not 0 <= l < self._n:
            raise IndexError(l)
        return self._fn(l)
