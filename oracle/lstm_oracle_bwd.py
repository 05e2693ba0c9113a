"""Plain fp64 CPU oracle of the stacked-LSTM backward pass (backpropagation through time).

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` may import or call this module.  It
shares no code with the HIP path; its forward half is the forward oracle's
definition written out again so that every step keeps the values the chain
rule needs.

What is computed.  For a scalar loss whose gradients with respect to the
forward outputs are given -- dy = dloss/dy [T, B, H], dhT = dloss/dhT and
dcT = dloss/dcT [L, B, H] (None: zero) -- the gradients with respect to every
input of the forward pass (x, h0, c0, and per layer W_l, R_l, b_l).  The
forward pass is the standard forget-gate LSTM of the forward oracle
(p = W_l u_t + R_l h_{t-1} + b_l, gate blocks i, f, g, o; c_t = f c_{t-1} + i g;
h_t = o tanh(c_t)).  The chain rule through it, per layer from the top down
and per step from the last to the first, with dh_rec = dloss/dh_t through
step t+1 (dhT[l] at the last step) and dc_rec = dloss/dc_t through c_{t+1}
(dcT[l] at the last step):

    dh    = dY_l[t] + dh_rec              (dY_l: dy for the top layer, else the
                                           input gradient of the layer above)
    dc    = dh o (1 - tanh(c_t)^2) + dc_rec
    dp_i  = dc g i (1 - i)      dp_f = dc c_{t-1} f (1 - f)
    dp_g  = dc i (1 - g^2)      dp_o = dh tanh(c_t) o (1 - o)
    dW_l += dp^T u_t     dR_l += dp^T h_{t-1}     db_l += sum over the batch of dp
    dU[t] = dp W_l       (dloss/du_t: the layer below's dY, or dx for layer 0)
    dh_rec = dp R_l      dc_rec = dc f
and dh0[l] = dh_rec, dc0[l] = dc_rec after the first step.  The weight
gradients are sums over all steps of products of per-step factors, so once
every step's dp is known they are single matrix products over all T*B columns
("Optimizing Performance of Recurrent Neural Networks on GPUs", proposed
method: the weight update done as one large product; the backward pass of
the layer below can run as soon as a layer's input gradients exist).  Here
they are accumulated step by step, as the definition reads.

Parity status: pinned by the CPU tests against central finite differences of
a 40-digit forward evaluation, against torch.autograd through torch.nn.LSTM in
float64, and by an exact saturation case; planted mistakes must fail a pin.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .lstm_oracle import sigmoid


def lstm_layer_saved(W: np.ndarray, R: np.ndarray, b: np.ndarray, U: np.ndarray, h0: np.ndarray,
                     c0: np.ndarray) -> Dict[str, np.ndarray]:
    """Forward of one layer over U [T, B, I_l] keeping what the backward pass needs:
    the activated gates i, f, g, o [T, B, H] each, c [T+1, B, H] (c[0] = c0) and
    h [T+1, B, H] (h[0] = h0)."""
    T = U.shape[0]
    B, H = h0.shape
    gi, gf, gg, go = (np.empty((T, B, H)) for _ in range(4))
    c = np.empty((T + 1, B, H))
    h = np.empty((T + 1, B, H))
    c[0], h[0] = c0, h0
    for t in range(T):
        p = U[t] @ W.T + h[t] @ R.T + b
        gi[t] = sigmoid(p[:, 0:H])
        gf[t] = sigmoid(p[:, H:2 * H])
        gg[t] = np.tanh(p[:, 2 * H:3 * H])
        go[t] = sigmoid(p[:, 3 * H:4 * H])
        c[t + 1] = gf[t] * c[t] + gi[t] * gg[t]
        h[t + 1] = go[t] * np.tanh(c[t + 1])
    return {"i": gi, "f": gf, "g": gg, "o": go, "c": c, "h": h}


def lstm_layer_backward(W: np.ndarray, R: np.ndarray, U: np.ndarray, s: Dict[str, np.ndarray], dY: np.ndarray,
                        dhT: Optional[np.ndarray], dcT: Optional[np.ndarray]) -> Dict[str, np.ndarray]:
    """Backward of one layer (see the module docstring).  dY: [T, B, H]; dhT, dcT: [B, H] or None.
    Returns dU [T, B, I_l], dW, dR, db, dh0, dc0."""
    T, B, H = dY.shape
    dW = np.zeros_like(W)
    dR = np.zeros_like(R)
    db = np.zeros(4 * H)
    dU = np.empty((T, B, W.shape[1]))
    dh_rec = np.zeros((B, H)) if dhT is None else np.asarray(dhT, dtype=np.float64).copy()
    dc_rec = np.zeros((B, H)) if dcT is None else np.asarray(dcT, dtype=np.float64).copy()
    for t in range(T - 1, -1, -1):
        i, f, g, o = s["i"][t], s["f"][t], s["g"][t], s["o"][t]
        c_prev, c_t, h_prev = s["c"][t], s["c"][t + 1], s["h"][t]
        tc = np.tanh(c_t)
        dh = dY[t] + dh_rec
        dc = dh * o * (1.0 - tc * tc) + dc_rec
        dp = np.concatenate([dc * g * i * (1.0 - i),
                             dc * c_prev * f * (1.0 - f),
                             dc * i * (1.0 - g * g),
                             dh * tc * o * (1.0 - o)], axis=1)   # [B, 4H], gate blocks i, f, g, o
        dW += dp.T @ U[t]
        dR += dp.T @ h_prev
        db += dp.sum(axis=0)
        dU[t] = dp @ W
        dh_rec = dp @ R
        dc_rec = dc * f
    return {"dU": dU, "dW": dW, "dR": dR, "db": db, "dh0": dh_rec, "dc0": dc_rec}


def lstm_backward(x: np.ndarray, W: Sequence[np.ndarray], R: Sequence[np.ndarray], b: Sequence[np.ndarray],
                  h0: Optional[np.ndarray], c0: Optional[np.ndarray], dy: np.ndarray,
                  dhT: Optional[np.ndarray] = None, dcT: Optional[np.ndarray] = None) -> Dict[str, object]:
    """Gradients of the stacked LSTM in fp64.

    Forward shapes as lstm_forward (x [T, B, I], W[l] [4H, I_l], R[l] [4H, H],
    b[l] [4H], h0 / c0 [L, B, H] or None); dy [T, B, H]; dhT / dcT [L, B, H] or
    None.  Returns {"dx": [T, B, I], "dh0": [L, B, H], "dc0": [L, B, H],
    "dW": [per layer], "dR": [per layer], "db": [per layer]} in fp64.
    """
    L = len(W)
    x64 = np.asarray(x, dtype=np.float64)
    T, B, _ = x64.shape
    H = np.asarray(R[0]).shape[1]
    Ws = [np.asarray(W[l], dtype=np.float64) for l in range(L)]
    Rs = [np.asarray(R[l], dtype=np.float64) for l in range(L)]
    bs = [np.asarray(b[l], dtype=np.float64) for l in range(L)]
    saved: List[Dict[str, np.ndarray]] = []
    inputs: List[np.ndarray] = []
    U = x64
    for l in range(L):
        hl = np.zeros((B, H)) if h0 is None else np.asarray(h0[l], dtype=np.float64)
        cl = np.zeros((B, H)) if c0 is None else np.asarray(c0[l], dtype=np.float64)
        s = lstm_layer_saved(Ws[l], Rs[l], bs[l], U, hl, cl)
        saved.append(s)
        inputs.append(U)
        U = s["h"][1:]
    dW: List[Optional[np.ndarray]] = [None] * L
    dR: List[Optional[np.ndarray]] = [None] * L
    db: List[Optional[np.ndarray]] = [None] * L
    dh0 = np.empty((L, B, H))
    dc0 = np.empty((L, B, H))
    dY = np.asarray(dy, dtype=np.float64)
    for l in range(L - 1, -1, -1):
        g = lstm_layer_backward(Ws[l], Rs[l], inputs[l], saved[l], dY,
                                None if dhT is None else dhT[l], None if dcT is None else dcT[l])
        dW[l], dR[l], db[l] = g["dW"], g["dR"], g["db"]
        dh0[l], dc0[l] = g["dh0"], g["dc0"]
        dY = g["dU"]
    return {"dx": dY, "dh0": dh0, "dc0": dc0, "dW": dW, "dR": dR, "db": db}


def lstm_backward_inputs(inp, dy: np.ndarray, dhT: Optional[np.ndarray] = None,
                         dcT: Optional[np.ndarray] = None) -> Dict[str, object]:
    """lstm_backward on an LSTM ``lstm_inputs.Inputs`` object (exact stored values, widened to fp64)."""
    if inp.cfg.cell != "lstm":
        raise ValueError("the backward oracle covers the LSTM cell")
    L = inp.cfg.L
    return lstm_backward(inp.x_f32(), [inp.W_f32(l) for l in range(L)], [inp.R_f32(l) for l in range(L)],
                         [inp.b_f32(l) for l in range(L)], inp.h0_f32(), inp.c0_f32(), dy, dhT, dcT)
