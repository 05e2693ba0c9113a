"""Pins that fix the fp64 oracle's GRU and simple-RNN cells against what their
definitions fix (the pages name the cells -- "Optimizing Performance of
Recurrent Neural Networks on GPUs", proposed method, last item: GRU with three
matrix groups, the simple RNN with one -- and print no equations, outputs or
examples, so every pin comes from the mathematics):

  Q1  torch.nn.GRU / torch.nn.RNN (tanh and relu) in float64 on the CPU,
      independent implementations of the same cells (GRU biases: bias_ih =
      b_r, b_z, b_Wn and bias_hh = 0, 0, b_Rn).
  Q2  brute-force memoised recursion over (layer, step), scalar loops, 40 digits,
      written from the definition independently of the oracle.
  Q3  special cases with a closed form: a GRU whose update gate saturates open
      (z = 1) carries h0 bit for bit; with z = 0 and r = 0 it reduces to
      tanh(W_n u + b_Wn), independent of h and R; a simple RNN with R = 0 is
      act(W x_t + b) per step; relu outputs are never negative.
  Q4  invariants: layer composition and time split (bitwise).
"""
from __future__ import annotations

import functools

import mpmath
import numpy as np

import lstm_inputs as li
import oracle.lstm_oracle as orc
from tests.pins import rel_err


def _msig(z):
    return 1 / (1 + mpmath.exp(-z))


def rand_params(cell, L=2, I=3, H=4, B=3, T=5, seed=1, scale=0.8, with_state=True):
    G, NB = li.ROWS[cell]
    rng = np.random.default_rng(seed)
    W = [rng.uniform(-scale, scale, (G * H, I if l == 0 else H)) for l in range(L)]
    R = [rng.uniform(-scale, scale, (G * H, H)) for _ in range(L)]
    b = [rng.uniform(-scale, scale, NB * H) for _ in range(L)]
    x = rng.standard_normal((T, B, I)) * 1.5
    h0 = rng.uniform(-1, 1, (L, B, H)) if with_state else None
    return x, W, R, b, h0


# ----------------------------------------------------------------------------- Q1
def torch_cell_f64(cell, x, W, R, b, h0=None):
    """torch.nn.GRU / RNN in float64 on the CPU with our weights."""
    import torch

    T, B, I = x.shape
    L = len(W)
    H = R[0].shape[1]
    if cell == "gru":
        m = torch.nn.GRU(I, H, num_layers=L).double()
    else:
        m = torch.nn.RNN(I, H, num_layers=L, nonlinearity="relu" if cell == "rnn_relu" else "tanh").double()
    with torch.no_grad():
        for l in range(L):
            getattr(m, f"weight_ih_l{l}").copy_(torch.from_numpy(np.asarray(W[l], dtype=np.float64)))
            getattr(m, f"weight_hh_l{l}").copy_(torch.from_numpy(np.asarray(R[l], dtype=np.float64)))
            bl = np.asarray(b[l], dtype=np.float64)
            if cell == "gru":
                bih = bl[:3 * H]
                bhh = np.concatenate([np.zeros(2 * H), bl[3 * H:]])
            else:
                bih, bhh = bl, np.zeros(H)
            getattr(m, f"bias_ih_l{l}").copy_(torch.from_numpy(bih))
            getattr(m, f"bias_hh_l{l}").copy_(torch.from_numpy(bhh))
        hz = torch.zeros(L, B, H, dtype=torch.float64) if h0 is None else torch.from_numpy(np.asarray(h0, dtype=np.float64))
        y, hT = m(torch.from_numpy(np.asarray(x, dtype=np.float64)), hz)
    return y.numpy(), hT.numpy()


def check_q1(cell, **kw):
    x, W, R, b, h0 = rand_params(cell, **kw)
    yt, ht = torch_cell_f64(cell, x, W, R, b, h0)
    y, hT, cT = orc.rnn_forward(cell, x, W, R, b, h0)
    assert cT is None
    return max(rel_err(y, yt), rel_err(hT, ht)), 1e-12


def check_q1_inputs(inp):
    """Q1 on a stored workload (exact values widened to fp64)."""
    L = inp.cfg.L
    x = inp.x_f32().astype(np.float64)
    W = [inp.W_f32(l).astype(np.float64) for l in range(L)]
    R = [inp.R_f32(l).astype(np.float64) for l in range(L)]
    b = [inp.b_f32(l).astype(np.float64) for l in range(L)]
    h0 = inp.h0_f32()
    yt, ht = torch_cell_f64(inp.cfg.cell, x, W, R, b, h0)
    y, hT, _ = orc.forward_inputs(inp)
    return max(rel_err(y, yt), rel_err(hT, ht)), 1e-12


# ----------------------------------------------------------------------------- Q2
def brute_force_cell(cell, x, W, R, b, h0=None, dps=40):
    """Memoised recursion state(l, t) -> h with scalar loops only, in mpmath."""
    mpmath.mp.dps = dps
    T, B = len(x), len(x[0])
    L = len(W)
    H = len(R[0][0])

    def dot(row, v):
        s = mpmath.mpf(0)
        for m in range(len(v)):
            s += mpmath.mpf(row[m]) * v[m]
        return s

    @functools.lru_cache(maxsize=None)
    def state(l, t):
        if t == 0:
            return tuple(tuple(mpmath.mpf(0 if h0 is None else h0[l][bb][j]) for j in range(H)) for bb in range(B))
        hp = state(l, t - 1)
        u = [[mpmath.mpf(v) for v in x[t - 1][bb]] for bb in range(B)] if l == 0 else state(l - 1, t)
        out = []
        for bb in range(B):
            row = []
            for j in range(H):
                if cell == "gru":
                    ar = dot(W[l][j], u[bb]) + dot(R[l][j], hp[bb]) + mpmath.mpf(b[l][j])
                    az = dot(W[l][H + j], u[bb]) + dot(R[l][H + j], hp[bb]) + mpmath.mpf(b[l][H + j])
                    rg, zg = _msig(ar), _msig(az)
                    ng = mpmath.tanh(dot(W[l][2 * H + j], u[bb]) + mpmath.mpf(b[l][2 * H + j]) +
                                     rg * (dot(R[l][2 * H + j], hp[bb]) + mpmath.mpf(b[l][3 * H + j])))
                    row.append((1 - zg) * ng + zg * hp[bb][j])
                else:
                    a = dot(W[l][j], u[bb]) + dot(R[l][j], hp[bb]) + mpmath.mpf(b[l][j])
                    row.append(mpmath.tanh(a) if cell == "rnn_tanh" else (a if a > 0 else mpmath.mpf(0)))
            out.append(tuple(row))
        return tuple(out)

    y = [[[state(L - 1, t + 1)[bb][j] for j in range(H)] for bb in range(B)] for t in range(T)]
    hT = [state(l, T) for l in range(L)]
    to = lambda a: np.array([[[float(v) for v in row] for row in m] for m in a])  # noqa: E731
    return to(y), to(hT)


def check_q2(cell, L=2, I=2, H=3, B=2, T=3, seed=5):
    x, W, R, b, h0 = rand_params(cell, L=L, I=I, H=H, B=B, T=T, seed=seed)
    yb, hb = brute_force_cell(cell, x.tolist(), [w.tolist() for w in W], [r.tolist() for r in R],
                              [v.tolist() for v in b], h0.tolist())
    y, hT, _ = orc.rnn_forward(cell, x, W, R, b, h0)
    return max(rel_err(y, yb), rel_err(hT, hb)), 1e-13


# ----------------------------------------------------------------------------- Q3
def check_q3_gru_update_gate_open():
    """b_z = +1e4: z = 1 exactly, so h_t = h0 bit for bit at every step and layer."""
    x, W, R, b, h0 = rand_params("gru", L=2, I=3, H=4, B=3, T=6, seed=9)
    H = 4
    for bl in b:
        bl[H:2 * H] = 1e4
    y, hT, _ = orc.rnn_forward("gru", x, W, R, b, h0)
    return bool(np.array_equal(hT, h0) and np.array_equal(y, np.broadcast_to(h0[-1], y.shape)))


def check_q3_gru_reset_and_update_closed():
    """b_z = b_r = -1e4: z = r = 0, so h_t = tanh(W_n u_t + b_Wn) whatever h and R are."""
    x, W, R, b, h0 = rand_params("gru", L=1, I=3, H=4, B=3, T=5, seed=4)
    H = 4
    b[0][0:2 * H] = -1e4
    y, _, _ = orc.rnn_forward("gru", x, W, R, b, h0)
    ref = np.tanh(x @ W[0][2 * H:3 * H].T + b[0][2 * H:3 * H])
    R2 = [r * -3.0 for r in R]
    y2, _, _ = orc.rnn_forward("gru", x, W, R2, b, h0 * 0.5)
    return max(rel_err(y, ref), rel_err(y2, ref)), 1e-15


def check_q3_rnn_zero_recurrence(cell):
    """R = 0: every step is act(W x_t + b) on its own."""
    x, W, R, b, h0 = rand_params(cell, L=1, I=3, H=4, B=3, T=5, seed=8)
    y, hT, _ = orc.rnn_forward(cell, x, W, [np.zeros_like(R[0])], b, h0)
    p = x @ W[0].T + b[0]
    ref = np.maximum(p, 0.0) if cell == "rnn_relu" else np.tanh(p)
    ok_sign = cell != "rnn_relu" or bool(np.all(y >= 0))
    return max(rel_err(y, ref), rel_err(hT[0], ref[-1])), 1e-15, ok_sign


# ----------------------------------------------------------------------------- Q4
def check_q4_layer_composition(cell):
    x, W, R, b, h0 = rand_params(cell, L=3, I=4, H=5, B=2, T=4, seed=3)
    y, hT, _ = orc.rnn_forward(cell, x, W, R, b, h0)
    U = x
    for l in range(3):
        U, h, _ = orc.rnn_forward(cell, U, W[l:l + 1], R[l:l + 1], b[l:l + 1], h0[l:l + 1])
        if not np.array_equal(h[0], hT[l]):
            return False
    return bool(np.array_equal(U, y))


def check_q4_time_split(cell, T1=2):
    x, W, R, b, h0 = rand_params(cell, L=2, I=4, H=5, B=2, T=5, seed=6)
    y, hT, _ = orc.rnn_forward(cell, x, W, R, b, h0)
    ya, ha, _ = orc.rnn_forward(cell, x[:T1], W, R, b, h0)
    yb, hb, _ = orc.rnn_forward(cell, x[T1:], W, R, b, ha)
    return bool(np.array_equal(np.concatenate([ya, yb]), y) and np.array_equal(hb, hT))
