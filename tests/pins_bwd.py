"""Pins that fix the fp64 backward oracle against what the LSTM definition fixes.

The pages give no formula, example or bound for the backward pass; these pins
come from the forward definition and from calculus:

  B1  central finite differences of the loss  sum(dy*y) + sum(dhT*hT) + sum(dcT*cT)
      with respect to every input element (x, h0, c0, W_l, R_l, b_l), the
      forward evaluated from the definition with scalar loops in 40-digit
      arithmetic (independent of both oracles), step 1e-15: the truncation error
      is ~1e-30, far below the fp64 gradients' own rounding;
  B2  torch.autograd through torch.nn.LSTM in float64 on the CPU (a library
      routine whose cell is the same definition: weight_ih = W, weight_hh = R,
      bias_ih = b, bias_hh = 0);
  B3  forget gate saturated open and input gate shut (b_f = +1e4, b_i = -1e4):
      with dy = dhT = 0 every gate derivative factor is exactly zero, so dc0
      equals dcT bit for bit and every other gradient is exactly zero.

Nothing here imports the HIP path.
"""
from __future__ import annotations

import mpmath
import numpy as np

import oracle.lstm_oracle_bwd as orcb
from tests.pins import rel_err


def _rand_problem(L, I, H, B, T, seed):
    rng = np.random.default_rng(seed)
    W = [rng.uniform(-0.8, 0.8, (4 * H, I if l == 0 else H)) for l in range(L)]
    R = [rng.uniform(-0.8, 0.8, (4 * H, H)) for _ in range(L)]
    b = [rng.uniform(-0.5, 0.5, 4 * H) for _ in range(L)]
    x = rng.standard_normal((T, B, I))
    h0 = rng.uniform(-0.6, 0.6, (L, B, H))
    c0 = rng.uniform(-0.6, 0.6, (L, B, H))
    dy = rng.standard_normal((T, B, H))
    dhT = rng.standard_normal((L, B, H))
    dcT = rng.standard_normal((L, B, H))
    return x, W, R, b, h0, c0, dy, dhT, dcT


# ----------------------------------------------------------------------------- B1
def mp_loss(x, W, R, b, h0, c0, dy, dhT, dcT):
    """The linear functional of the forward outputs, in mpmath (values are mpf
    or float nested lists); the forward is written out from the definition."""
    sig = lambda z: 1 / (1 + mpmath.exp(-z))  # noqa: E731
    L = len(W)
    T, B = len(x), len(x[0])
    H = len(R[0][0])
    U = [[[mpmath.mpf(v) for v in x[t][bb]] for bb in range(B)] for t in range(T)]
    loss = mpmath.mpf(0)
    for l in range(L):
        h = [[mpmath.mpf(h0[l][bb][j]) for j in range(H)] for bb in range(B)]
        c = [[mpmath.mpf(c0[l][bb][j]) for j in range(H)] for bb in range(B)]
        Y = []
        for t in range(T):
            hn = [[None] * H for _ in range(B)]
            cn = [[None] * H for _ in range(B)]
            for bb in range(B):
                for j in range(H):
                    p = []
                    for k in range(4):
                        row = k * H + j
                        s = mpmath.mpf(b[l][row])
                        for m in range(len(U[t][bb])):
                            s += mpmath.mpf(W[l][row][m]) * U[t][bb][m]
                        for m in range(H):
                            s += mpmath.mpf(R[l][row][m]) * h[bb][m]
                        p.append(s)
                    cc = sig(p[1]) * c[bb][j] + sig(p[0]) * mpmath.tanh(p[2])
                    cn[bb][j] = cc
                    hn[bb][j] = sig(p[3]) * mpmath.tanh(cc)
            h, c = hn, cn
            Y.append(h)
        for bb in range(B):
            for j in range(H):
                loss += mpmath.mpf(dhT[l][bb][j]) * h[bb][j] + mpmath.mpf(dcT[l][bb][j]) * c[bb][j]
        U = Y
    for t in range(T):
        for bb in range(B):
            for j in range(H):
                loss += mpmath.mpf(dy[t][bb][j]) * U[t][bb][j]
    return loss


def check_b1(L=2, I=3, H=2, B=2, T=3, seed=21, eps="1e-15"):
    """Max relative error of every oracle gradient against 40-digit central differences."""
    mpmath.mp.dps = 40
    x, W, R, b, h0, c0, dy, dhT, dcT = _rand_problem(L, I, H, B, T, seed)
    g = orcb.lstm_backward(x, W, R, b, h0, c0, dy, dhT, dcT)
    h = mpmath.mpf(eps)
    base = {"x": x.tolist(), "W": [w.tolist() for w in W], "R": [r.tolist() for r in R],
            "b": [v.tolist() for v in b], "h0": h0.tolist(), "c0": c0.tolist()}

    def fd(name, path):
        def perturbed(delta):
            args = {k: (v if k != name else _set(v, path, delta)) for k, v in base.items()}
            return mp_loss(args["x"], args["W"], args["R"], args["b"], args["h0"], args["c0"],
                           dy.tolist(), dhT.tolist(), dcT.tolist())
        return float((perturbed(h) - perturbed(-h)) / (2 * h))

    worst = 0.0
    for name, grad in (("x", g["dx"]), ("h0", g["dh0"]), ("c0", g["dc0"])):
        ref = np.array([fd(name, idx) for idx in np.ndindex(grad.shape)]).reshape(grad.shape)
        worst = max(worst, rel_err(grad, ref))
    for name, key in (("W", "dW"), ("R", "dR"), ("b", "db")):
        for l in range(L):
            grad = g[key][l]
            ref = np.array([fd(name, (l,) + idx) for idx in np.ndindex(grad.shape)]).reshape(grad.shape)
            worst = max(worst, rel_err(grad, ref))
    return worst, 1e-12


def _set(nested, path, delta):
    """Copy of a nested list with element `path` shifted by the mpf `delta`."""
    if len(path) == 1:
        out = list(nested)
        out[path[0]] = mpmath.mpf(out[path[0]]) + delta
        return out
    out = list(nested)
    out[path[0]] = _set(nested[path[0]], path[1:], delta)
    return out


# ----------------------------------------------------------------------------- B2
def torch_grads(x, W, R, b, h0, c0, dy, dhT, dcT):
    """Gradients of the same loss through torch.nn.LSTM in float64 (CPU)."""
    import torch
    T, B, I = x.shape
    L = len(W)
    H = R[0].shape[1]
    m = torch.nn.LSTM(I, H, num_layers=L).double()
    with torch.no_grad():
        for l in range(L):
            getattr(m, f"weight_ih_l{l}").copy_(torch.from_numpy(W[l]))
            getattr(m, f"weight_hh_l{l}").copy_(torch.from_numpy(R[l]))
            getattr(m, f"bias_ih_l{l}").copy_(torch.from_numpy(b[l]))
            getattr(m, f"bias_hh_l{l}").zero_()
    xt = torch.from_numpy(x).clone().requires_grad_(True)
    ht = torch.from_numpy(h0).clone().requires_grad_(True)
    ct = torch.from_numpy(c0).clone().requires_grad_(True)
    y, (hT, cT) = m(xt, (ht, ct))
    loss = (y * torch.from_numpy(dy)).sum() + (hT * torch.from_numpy(dhT)).sum() + (cT * torch.from_numpy(dcT)).sum()
    loss.backward()
    return {"dx": xt.grad.numpy(), "dh0": ht.grad.numpy(), "dc0": ct.grad.numpy(),
            "dW": [getattr(m, f"weight_ih_l{l}").grad.numpy() for l in range(L)],
            "dR": [getattr(m, f"weight_hh_l{l}").grad.numpy() for l in range(L)],
            "db": [getattr(m, f"bias_ih_l{l}").grad.numpy() for l in range(L)],
            "db_hh": [getattr(m, f"bias_hh_l{l}").grad.numpy() for l in range(L)]}


def check_b2(L=3, I=5, H=4, B=3, T=6, seed=22):
    x, W, R, b, h0, c0, dy, dhT, dcT = _rand_problem(L, I, H, B, T, seed)
    g = orcb.lstm_backward(x, W, R, b, h0, c0, dy, dhT, dcT)
    t = torch_grads(x, W, R, b, h0, c0, dy, dhT, dcT)
    worst = max(rel_err(g[k], t[k]) for k in ("dx", "dh0", "dc0"))
    for k in ("dW", "dR", "db"):
        worst = max(worst, max(rel_err(g[k][l], t[k][l]) for l in range(L)))
    # the single bias is the sum of torch's two: both get the same gradient
    worst = max(worst, max(rel_err(g["db"][l], t["db_hh"][l]) for l in range(L)))
    return worst, 1e-12


# ----------------------------------------------------------------------------- B3
def check_b3(L=2, I=4, H=3, B=2, T=5, seed=23):
    """Returns True when the saturated case is exact: dc0 == dcT bitwise, all else zero."""
    x, W, R, b, h0, c0, _, _, dcT = _rand_problem(L, I, H, B, T, seed)
    for bl in b:
        bl[0:H] = -1e4      # input gate shut
        bl[H:2 * H] = 1e4   # forget gate open
    zeros = np.zeros((T, B, H))
    g = orcb.lstm_backward(x, W, R, b, h0, c0, zeros, np.zeros((L, B, H)), dcT)
    ok = np.array_equal(g["dc0"], dcT)
    ok &= not np.any(g["dx"]) and not np.any(g["dh0"])
    for l in range(L):
        ok &= not np.any(g["dW"][l]) and not np.any(g["dR"][l]) and not np.any(g["db"][l])
    return bool(ok)
