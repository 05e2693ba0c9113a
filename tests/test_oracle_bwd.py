"""CPU tests that pin the fp64 backward oracle (oracle/lstm_oracle_bwd.py):
B1 finite differences at 40 digits, B2 torch.autograd in float64, B3 exact
saturation; and planted mistakes in the oracle that must each fail a pin."""
import numpy as np
import pytest

import oracle.lstm_oracle_bwd as orcb
import tests.pins_bwd as pb


def test_b1_finite_differences():
    err, bound = pb.check_b1()
    assert err <= bound, err


def test_b1_finite_differences_single_layer_wide_input():
    err, bound = pb.check_b1(L=1, I=4, H=3, B=1, T=4, seed=31)
    assert err <= bound, err


def test_b2_torch_autograd():
    err, bound = pb.check_b2()
    assert err <= bound, err


def test_b2_torch_autograd_workload_like():
    """A 4-layer I = H = 64 stack, B = 8, T = 10 (the oracle's products at scale)."""
    err, bound = pb.check_b2(L=4, I=64, H=64, B=8, T=10, seed=24)
    assert err <= bound, err


def test_b3_saturation_exact():
    assert pb.check_b3()


# ----------------------------------------------------------------------------- planted mistakes
def _mutant(kind):
    def layer_backward(W, R, U, s, dY, dhT, dcT):
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
            dct = (1.0 - tc * tc) if kind != "no_tanh_derivative" else 1.0
            dc = dh * o * dct + dc_rec
            cf = c_t if kind == "c_t_in_forget" else c_prev
            gi, gg = (g, i) if kind != "swap_i_g" else (i, g)
            dp = np.concatenate([dc * gi * i * (1.0 - i), dc * cf * f * (1.0 - f),
                                 dc * gg * (1.0 - g * g), dh * tc * o * (1.0 - o)], axis=1)
            dW += dp.T @ (U[t] if kind != "no_input_in_dW" else np.zeros_like(U[t]))
            dR += dp.T @ (h_prev if kind != "h_t_in_dR" else s["h"][t + 1])
            db += dp.sum(axis=0) if kind != "bias_one_row" else dp[0]
            dU[t] = dp @ W if kind != "no_input_gradient" else 0.0
            dh_rec = dp @ R
            dc_rec = dc * f if kind != "no_forget_in_dc" else dc
        return {"dU": dU, "dW": dW, "dR": dR, "db": db, "dh0": dh_rec, "dc0": dc_rec}
    return layer_backward


def _pins_pass():
    try:
        for chk in (pb.check_b1, pb.check_b2):
            err, bound = chk()
            if not err <= bound:
                return False
        return pb.check_b3()
    except Exception:  # a shape error is a failed pin too
        return False


@pytest.mark.parametrize("kind", ["no_tanh_derivative", "c_t_in_forget", "swap_i_g", "no_input_in_dW",
                                  "h_t_in_dR", "bias_one_row", "no_input_gradient", "no_forget_in_dc"])
def test_backward_pins_catch_mutations(monkeypatch, kind):
    assert _pins_pass(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(orcb, "lstm_layer_backward", _mutant(kind))
    assert not _pins_pass(), f"mutation {kind} was not caught by any pin"
