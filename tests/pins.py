"""Pins that fix the fp64 oracle against what the LSTM definition itself fixes.

The pages print no worked example, table of outputs or error bound, so every
pin here comes from the mathematics of the standard forget-gate LSTM (one
grouped 4H-row product per weight matrix, gate blocks i, f, g, o; "Optimizing
Performance of Recurrent Neural Networks on GPUs", proposed method):

  P1  H = I = B = L = 1 closed form, evaluated step by step in 40-digit arithmetic.
  P2  zero x and zero R: every (b, j) is an affine scalar recursion with constant
      gates, c_t = c* + f^t (c0 - c*), c* = i g / (1 - f), h_t = o tanh(c_t).
  P3  forget bias -> +inf, input bias -> -inf: c is carried bit-exactly.
  P4  brute-force memoised recursion over (layer, step), scalar loops, 40 digits.
  P5  torch.nn.LSTM in float64 on the CPU (weight_ih = W, weight_hh = R,
      bias_ih = b, bias_hh = 0), a library routine that reduces to the same definition.
  P6  invariants: layer composition, time split, batch permutation, bounds.

Each ``check_*`` returns a (max error, bound) pair or raises; the tests assert,
and ``test_pins_catch_mutations`` plants mistakes in the oracle and requires
that some pin fails.  Nothing here imports the HIP path.
"""
from __future__ import annotations

import functools
import math

import mpmath
import numpy as np

import lstm_inputs as li
import oracle.lstm_oracle as orc

mpmath.mp.dps = 40


# ----------------------------------------------------------------------------- helpers
def rel_err(a: np.ndarray, r: np.ndarray) -> float:
    """Max-norm relative error ||a - r||_inf / ||r||_inf (||a||_inf if r is all zero)."""
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = float(np.max(np.abs(r))) if r.size else 0.0
    num = float(np.max(np.abs(a - r))) if r.size else 0.0
    if den == 0.0:
        den = float(np.max(np.abs(a))) if a.size else 0.0
        return num if den == 0.0 else num / den
    return num / den


def _msig(z):
    return 1 / (1 + mpmath.exp(-z))


# ----------------------------------------------------------------------------- P1
P1_W = [0.5, -0.25, 1.0, 0.75]      # rows i, f, g, o of the 4x1 input matrix
P1_R = [0.1, 0.2, -0.3, 0.4]
P1_B = [0.0, 1.0, 0.0, -0.5]
P1_X = [1.0, -1.0, 0.5]


def p1_closed_form():
    """Scalar LSTM, every gate with a distinct weight, written out in 40-digit arithmetic."""
    h = mpmath.mpf(0)
    c = mpmath.mpf(0)
    hs, cs, gates = [], [], []
    for x in P1_X:
        x = mpmath.mpf(x)
        p = [mpmath.mpf(P1_W[k]) * x + mpmath.mpf(P1_R[k]) * h + mpmath.mpf(P1_B[k]) for k in range(4)]
        i, f, g, o = _msig(p[0]), _msig(p[1]), mpmath.tanh(p[2]), _msig(p[3])
        c = f * c + i * g
        h = o * mpmath.tanh(c)
        hs.append(h)
        cs.append(c)
        gates.append((i, f, g, o))
    return hs, cs, gates


def check_p1():
    hs, cs, _ = p1_closed_form()
    x = np.array(P1_X, dtype=np.float64).reshape(3, 1, 1)
    W = [np.array(P1_W).reshape(4, 1)]
    R = [np.array(P1_R).reshape(4, 1)]
    b = [np.array(P1_B)]
    y, hT, cT = orc.lstm_forward(x, W, R, b)
    err = 0.0
    for t in range(3):
        err = max(err, abs((y[t, 0, 0] - float(hs[t])) / float(hs[t])))
    err = max(err, abs((cT[0, 0, 0] - float(cs[-1])) / float(cs[-1])))
    err = max(err, abs((hT[0, 0, 0] - float(hs[-1])) / float(hs[-1])))
    return err, 1e-15


# ----------------------------------------------------------------------------- P2
def check_p2(H=3, B=2, T=16, seed=7):
    """Zero x and zero R: closed-form affine recursion per (b, j)."""
    rng = np.random.default_rng(seed)
    I = 2
    W = [rng.uniform(-1, 1, (4 * H, I))]
    R = [np.zeros((4 * H, H))]
    b = [rng.uniform(-1.5, 1.5, 4 * H)]
    c0 = rng.uniform(-1, 1, (1, B, H))
    h0 = rng.uniform(-1, 1, (1, B, H))   # irrelevant because R = 0
    x = np.zeros((T, B, I))
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    err = 0.0
    for bb in range(B):
        for j in range(H):
            bi, bf, bg, bo = (mpmath.mpf(b[0][k * H + j]) for k in range(4))
            i, f, g, o = _msig(bi), _msig(bf), mpmath.tanh(bg), _msig(bo)
            cstar = i * g / (1 - f)
            for t in range(1, T + 1):
                ct = cstar + f ** t * (mpmath.mpf(c0[0, bb, j]) - cstar)
                ht = o * mpmath.tanh(ct)
                err = max(err, abs(float(y[t - 1, bb, j]) - float(ht)) / max(abs(float(ht)), 1e-300))
            err = max(err, abs(float(cT[0, bb, j]) - float(ct)) / abs(float(ct)))
    return err, 1e-13


def check_p2_constant_states():
    """b = 0, c0 = 0 gives c == h == 0 exactly; c0 = c* keeps c at c*."""
    H, B, T = 2, 2, 8
    x = np.zeros((T, B, 3))
    W = [np.ones((4 * H, 3))]
    R = [np.zeros((4 * H, H))]
    y, hT, cT = orc.lstm_forward(x, W, R, [np.zeros(4 * H)])
    exact_zero = bool(np.all(y == 0.0) and np.all(hT == 0.0) and np.all(cT == 0.0))
    # fixed point
    bvec = np.array([0.5, 0.5, 1.0, 1.0, -0.5, -0.5, 0.25, 0.25])
    i = 1 / (1 + math.exp(-0.5))
    f = 1 / (1 + math.exp(-1.0))
    g = math.tanh(-0.5)
    cstar = i * g / (1 - f)
    c0 = np.full((1, B, H), cstar)
    y2, _, cT2 = orc.lstm_forward(x, W, R, [bvec], None, c0)
    drift = float(np.max(np.abs(cT2 - cstar)))
    o = 1 / (1 + math.exp(-0.25))
    herr = float(np.max(np.abs(y2 - o * math.tanh(cstar))))
    return exact_zero, max(drift, herr)


def p2_worked_example():
    """b = [0.5, 1.0, -0.5, 0.25], c0 = 0.3, 16 steps: c*, c_16, h_16 in 40 digits."""
    i, f, g, o = _msig(mpmath.mpf("0.5")), _msig(mpmath.mpf(1)), mpmath.tanh(mpmath.mpf("-0.5")), _msig(mpmath.mpf("0.25"))
    cstar = i * g / (1 - f)
    c16 = cstar + f ** 16 * (mpmath.mpf("0.3") - cstar)
    return cstar, c16, o * mpmath.tanh(c16)


def check_p2_worked():
    cstar, c16, h16 = p2_worked_example()
    x = np.zeros((16, 1, 1))
    W = [np.zeros((4, 1))]
    R = [np.zeros((4, 1))]
    b = [np.array([0.5, 1.0, -0.5, 0.25])]
    y, hT, cT = orc.lstm_forward(x, W, R, b, None, np.full((1, 1, 1), 0.3))
    return max(abs(cT[0, 0, 0] - float(c16)) / abs(float(c16)),
               abs(y[-1, 0, 0] - float(h16)) / abs(float(h16))), 1e-14


# ----------------------------------------------------------------------------- P3
def saturating_inputs(L=2, I=5, H=4, B=3, T=6, seed=11):
    rng = np.random.default_rng(seed)
    W = [rng.uniform(-0.5, 0.5, (4 * H, I if l == 0 else H)) for l in range(L)]
    R = [rng.uniform(-0.5, 0.5, (4 * H, H)) for _ in range(L)]
    b = []
    for _ in range(L):
        bl = rng.uniform(-0.5, 0.5, 4 * H)
        bl[0:H] = -1e4          # input gate -> 0
        bl[H:2 * H] = 1e4       # forget gate -> 1
        b.append(bl)
    x = rng.standard_normal((T, B, I))
    c0 = rng.uniform(-1, 1, (L, B, H))
    h0 = rng.uniform(-1, 1, (L, B, H))
    return x, W, R, b, h0, c0


def check_p3():
    """cT == c0 bit for bit, and h_t = o_t tanh(c0) with o_t in (0, 1)."""
    x, W, R, b, h0, c0 = saturating_inputs()
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    bit_exact = bool(np.array_equal(cT, c0))
    ratio = hT / np.tanh(c0)
    in_range = bool(np.all(ratio > 0) and np.all(ratio < 1))
    return bit_exact, in_range


# ----------------------------------------------------------------------------- P4
def brute_force(x, W, R, b, h0=None, c0=None, dps=40):
    """Memoised recursion state(l, t) -> (h, c) with scalar loops only, in mpmath.

    x: [T][B][I] nested sequences; W[l]: [4H][I_l]; R[l]: [4H][H]; b[l]: [4H].
    Written from the definition, independently of the oracle.
    """
    mpmath.mp.dps = dps
    T, B = len(x), len(x[0])
    L = len(W)
    H = len(R[0][0])

    @functools.lru_cache(maxsize=None)
    def state(l, t):
        # returns (h, c) after t steps of layer l as tuples [B][H]
        if t == 0:
            h = tuple(tuple(mpmath.mpf(0 if h0 is None else h0[l][bb][j]) for j in range(H)) for bb in range(B))
            c = tuple(tuple(mpmath.mpf(0 if c0 is None else c0[l][bb][j]) for j in range(H)) for bb in range(B))
            return h, c
        hprev, cprev = state(l, t - 1)
        if l == 0:
            u = [[mpmath.mpf(v) for v in x[t - 1][bb]] for bb in range(B)]
        else:
            u = state(l - 1, t)[0]
        hn, cn = [], []
        for bb in range(B):
            hrow, crow = [], []
            for j in range(H):
                p = []
                for k in range(4):
                    row = k * H + j
                    s = mpmath.mpf(b[l][row])
                    for m in range(len(u[bb])):
                        s += mpmath.mpf(W[l][row][m]) * u[bb][m]
                    for m in range(H):
                        s += mpmath.mpf(R[l][row][m]) * hprev[bb][m]
                    p.append(s)
                ig, fg, gg, og = _msig(p[0]), _msig(p[1]), mpmath.tanh(p[2]), _msig(p[3])
                cc = fg * cprev[bb][j] + ig * gg
                crow.append(cc)
                hrow.append(og * mpmath.tanh(cc))
            hn.append(tuple(hrow))
            cn.append(tuple(crow))
        return tuple(hn), tuple(cn)

    y = [[[state(L - 1, t + 1)[0][bb][j] for j in range(H)] for bb in range(B)] for t in range(T)]
    hT = [state(l, T)[0] for l in range(L)]
    cT = [state(l, T)[1] for l in range(L)]
    to = lambda a: np.array([[[float(v) for v in row] for row in m] for m in a])  # noqa: E731
    return to(y), to(hT), to(cT)


def check_p4(L=3, I=2, H=3, B=2, T=4, seed=5, with_state=True):
    rng = np.random.default_rng(seed)
    W = [rng.uniform(-1, 1, (4 * H, I if l == 0 else H)) for l in range(L)]
    R = [rng.uniform(-1, 1, (4 * H, H)) for _ in range(L)]
    b = [rng.uniform(-1, 1, 4 * H) for _ in range(L)]
    x = rng.standard_normal((T, B, I))
    h0 = rng.uniform(-1, 1, (L, B, H)) if with_state else None
    c0 = rng.uniform(-1, 1, (L, B, H)) if with_state else None
    yb, hb, cb = brute_force(x.tolist(), [w.tolist() for w in W], [r.tolist() for r in R],
                             [v.tolist() for v in b],
                             None if h0 is None else h0.tolist(), None if c0 is None else c0.tolist())
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    return max(rel_err(y, yb), rel_err(hT, hb), rel_err(cT, cb)), 1e-13


# ----------------------------------------------------------------------------- P5
def torch_lstm_f64(x, W, R, b, h0=None, c0=None):
    """torch.nn.LSTM in float64 on the CPU with bias_hh = 0."""
    import torch

    T, B, I = x.shape
    L = len(W)
    H = R[0].shape[1]
    m = torch.nn.LSTM(I, H, num_layers=L).double()
    with torch.no_grad():
        for l in range(L):
            getattr(m, f"weight_ih_l{l}").copy_(torch.from_numpy(np.asarray(W[l], dtype=np.float64)))
            getattr(m, f"weight_hh_l{l}").copy_(torch.from_numpy(np.asarray(R[l], dtype=np.float64)))
            getattr(m, f"bias_ih_l{l}").copy_(torch.from_numpy(np.asarray(b[l], dtype=np.float64)))
            getattr(m, f"bias_hh_l{l}").zero_()
        hz = torch.zeros(L, B, H, dtype=torch.float64) if h0 is None else torch.from_numpy(np.asarray(h0, dtype=np.float64))
        cz = torch.zeros(L, B, H, dtype=torch.float64) if c0 is None else torch.from_numpy(np.asarray(c0, dtype=np.float64))
        y, (hT, cT) = m(torch.from_numpy(np.asarray(x, dtype=np.float64)), (hz, cz))
    return y.numpy(), hT.numpy(), cT.numpy()


def check_p5_inputs(inp, T_cut=None, B_cut=None, L_cut=None):
    L = inp.cfg.L if L_cut is None else min(L_cut, inp.cfg.L)
    x = inp.x_f32().astype(np.float64)
    h0, c0 = inp.h0_f32(), inp.c0_f32()
    if T_cut is not None:
        x = x[:T_cut]
    if B_cut is not None:
        x = x[:, :B_cut]
        h0 = None if h0 is None else h0[:, :B_cut]
        c0 = None if c0 is None else c0[:, :B_cut]
    if h0 is not None:
        h0, c0 = h0[:L], c0[:L]
    W = [inp.W_f32(l).astype(np.float64) for l in range(L)]
    R = [inp.R_f32(l).astype(np.float64) for l in range(L)]
    b = [inp.b_f32(l).astype(np.float64) for l in range(L)]
    yt, ht, ct = torch_lstm_f64(x, W, R, b, h0, c0)
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    return max(rel_err(y, yt), rel_err(hT, ht), rel_err(cT, ct)), 1e-12


# ----------------------------------------------------------------------------- P6
def p6_inputs(L=3, I=4, H=5, B=4, T=7, seed=3):
    rng = np.random.default_rng(seed)
    W = [rng.uniform(-0.6, 0.6, (4 * H, I if l == 0 else H)) for l in range(L)]
    R = [rng.uniform(-0.6, 0.6, (4 * H, H)) for _ in range(L)]
    b = [rng.uniform(-0.6, 0.6, 4 * H) for _ in range(L)]
    x = rng.standard_normal((T, B, I)) * 2
    h0 = rng.uniform(-1, 1, (L, B, H))
    c0 = rng.uniform(-1, 1, (L, B, H))
    return x, W, R, b, h0, c0


def check_p6_layer_composition():
    x, W, R, b, h0, c0 = p6_inputs()
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    U = x
    for l in range(len(W)):
        U, h1, c1 = orc.lstm_forward(U, [W[l]], [R[l]], [b[l]], h0[l:l + 1], c0[l:l + 1])
        if not (np.array_equal(h1[0], hT[l]) and np.array_equal(c1[0], cT[l])):
            return False
    return bool(np.array_equal(U, y))


def check_p6_time_split(T1=3):
    x, W, R, b, h0, c0 = p6_inputs()
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    ya, ha, ca = orc.lstm_forward(x[:T1], W, R, b, h0, c0)
    yb, hb, cb = orc.lstm_forward(x[T1:], W, R, b, ha, ca)
    return bool(np.array_equal(np.concatenate([ya, yb]), y) and np.array_equal(hb, hT) and np.array_equal(cb, cT))


def check_p6_batch_permutation():
    x, W, R, b, h0, c0 = p6_inputs()
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    perm = np.array([2, 0, 3, 1])
    yp, hp, cp = orc.lstm_forward(x[:, perm], W, R, b, h0[:, perm], c0[:, perm])
    single = orc.lstm_forward(x[:, 1:2], W, R, b, h0[:, 1:2], c0[:, 1:2])
    return max(rel_err(yp, y[:, perm]), rel_err(hp, hT[:, perm]), rel_err(cp, cT[:, perm]),
               rel_err(single[0], y[:, 1:2]), rel_err(single[2], cT[:, 1:2])), 1e-14


def check_p6_bounds():
    x, W, R, b, h0, c0 = p6_inputs()
    x = x * 10
    T = x.shape[0]
    y, hT, cT = orc.lstm_forward(x, W, R, b, h0, c0)
    return bool(np.all(np.abs(y) < 1) and np.all(np.abs(cT) <= np.abs(c0) + T))


def check_p6_recipe_bf16_exact():
    """bf16 workloads: the oracle must see the stored bf16 values exactly."""
    cfg = li.custom_config(1, 3, 2, 1, 1, "bf16")
    inp = li.make_inputs(cfg)
    w = inp.W_f32(0)
    back = li.bf16_bits_from_f32(w)
    return bool(np.array_equal(back, inp.W[0]))
