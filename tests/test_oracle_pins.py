"""CPU tests: the fp64 oracle against what the LSTM definition fixes (pins P1-P6).

See ``tests/pins.py`` for the derivation of each pin.  The last test plants
plausible mistakes in the oracle (on the CPU) and requires every one of them to
fail at least one pin.
"""
import json
import os

import mpmath
import numpy as np
import pytest

import lstm_inputs as li
import oracle.lstm_oracle as orc
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_sigmoid_saturates_exactly():
    z = np.array([-1e4, -800.0, -50.0, 0.0, 50.0, 800.0, 1e4])
    s = orc.sigmoid(z)
    assert s[0] == 0.0 and s[-1] == 1.0
    assert s[3] == 0.5
    np.testing.assert_allclose(s[2], np.exp(-50.0) / (1 + np.exp(-50.0)), rtol=1e-15)
    mp = [float(1 / (1 + mpmath.exp(-mpmath.mpf(v)))) for v in (-50.0, -3.5, 0.25, 7.0)]
    np.testing.assert_allclose(orc.sigmoid(np.array([-50.0, -3.5, 0.25, 7.0])), mp, rtol=1e-15)


def test_p1_scalar_closed_form():
    err, bound = pins.check_p1()
    assert err <= bound, err


def test_p1_golden_fixture_inputs():
    """The P1 inputs stored under tests/golden match the ones the pin evaluates."""
    with open(os.path.join(GOLDEN, "p1_scalar_lstm.json")) as f:
        g = json.load(f)
    assert g["W"] == pins.P1_W and g["R"] == pins.P1_R and g["b"] == pins.P1_B and g["x"] == pins.P1_X
    hs, cs, gates = pins.p1_closed_form()
    # the t = 1 gates follow from the inputs alone: i = s(0.5), f = s(0.75), g = tanh(1), o = s(0.25)
    i, f, gg, o = gates[0]
    assert abs(i - 1 / (1 + mpmath.exp(-0.5))) < 1e-35
    assert abs(f - 1 / (1 + mpmath.exp(-0.75))) < 1e-35
    assert abs(gg - mpmath.tanh(1)) < 1e-35
    assert abs(o - 1 / (1 + mpmath.exp(-0.25))) < 1e-35


def test_p2_zero_x_zero_R_closed_form():
    err, bound = pins.check_p2()
    assert err <= bound, err


def test_p2_constant_states():
    exact_zero, drift = pins.check_p2_constant_states()
    assert exact_zero
    assert drift < 1e-15


def test_p2_worked_example():
    err, bound = pins.check_p2_worked()
    assert err <= bound, err


def test_p3_saturation_carries_c_exactly():
    bit_exact, in_range = pins.check_p3()
    assert bit_exact and in_range


def test_p4_bruteforce_three_layers():
    err, bound = pins.check_p4()
    assert err <= bound, err


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (2, 3, 1, 2, 3), (1, 1, 3, 1, 2), (2, 2, 2, 2, 4)])
def test_p4_bruteforce_tiny_shapes(shape):
    L, I, H, B, T = shape
    err, bound = pins.check_p4(L=L, I=I, H=H, B=B, T=T, seed=sum(shape), with_state=(H % 2 == 0))
    assert err <= bound, err


@pytest.mark.parametrize("name,T_cut,B_cut,L_cut,rs", [
    ("c1", None, None, None, False),
    ("c1", None, None, None, True),
    ("c2", 8, None, None, False),
    ("c3", 8, None, None, True),
    ("c5", 8, None, None, False),
])
def test_p5_torch_lstm_float64(name, T_cut, B_cut, L_cut, rs):
    inp = li.make_inputs(li.CONFIGS[name], random_state=rs)
    err, bound = pins.check_p5_inputs(inp, T_cut=T_cut, B_cut=B_cut, L_cut=L_cut)
    assert err <= bound, err


@pytest.mark.slow
def test_p5_torch_lstm_float64_large_hidden():
    """The H = 4096 shape, first layer, two steps, two sequences."""
    cfg = li.CONFIGS["c4"]
    small = li.Config("c4-l1", cfg.cfg_id, 1, cfg.I, cfg.H, cfg.B, 2, cfg.dtype)
    inp = li.make_inputs(small)
    err, bound = pins.check_p5_inputs(inp, B_cut=2)
    assert err <= bound, err


def test_p6_layer_composition_bitwise():
    assert pins.check_p6_layer_composition()


def test_p6_time_split_bitwise():
    assert pins.check_p6_time_split()


def test_p6_batch_permutation():
    err, bound = pins.check_p6_batch_permutation()
    assert err <= bound, err


def test_p6_bounds():
    assert pins.check_p6_bounds()


def test_bf16_inputs_are_exact_for_oracle():
    assert pins.check_p6_recipe_bf16_exact()


# ----------------------------------------------------------------------------- mutations
def _all_pins_pass() -> bool:
    try:
        checks = [pins.check_p1(), pins.check_p2(H=2, B=1, T=5), pins.check_p2_worked(),
                  pins.check_p4(L=2, I=2, H=2, B=1, T=3)]
        if any(e > bnd for e, bnd in checks):
            return False
        z, drift = pins.check_p2_constant_states()
        if not z or drift > 1e-15:
            return False
        be, ir = pins.check_p3()
        if not (be and ir):
            return False
        if not (pins.check_p6_layer_composition() and pins.check_p6_time_split() and pins.check_p6_bounds()):
            return False
        return True
    except Exception:
        return False


def _mut_cell(kind):
    def cell(W, R, b, u, h, c):
        H = R.shape[1]
        if kind == "transpose_R":
            Rt = R.reshape(4, H, H).transpose(0, 2, 1).reshape(4 * H, H)
            p = u @ W.T + h @ Rt.T + b
        elif kind == "drop_bias":
            p = u @ W.T + h @ R.T
        elif kind == "drop_recurrent":
            p = u @ W.T + b
        else:
            p = u @ W.T + h @ R.T + b
        s = orc.sigmoid
        i, f, g, o = s(p[:, :H]), s(p[:, H:2 * H]), np.tanh(p[:, 2 * H:3 * H]), s(p[:, 3 * H:])
        if kind == "swap_if":
            i, f = f, i
        if kind == "swap_go":
            g, o = np.tanh(p[:, 3 * H:]), s(p[:, 2 * H:3 * H])
        if kind == "sigmoid_sign":
            o = s(-p[:, 3 * H:])
        c_new = f * c + i * g
        if kind == "forget_dropped":
            c_new = c + i * g
        h_new = o * np.tanh(c_new)
        if kind == "h_uses_old_c":
            h_new = o * np.tanh(c)
        return h_new, c_new
    return cell


@pytest.mark.parametrize("kind", ["transpose_R", "drop_bias", "drop_recurrent", "swap_if", "swap_go",
                                  "sigmoid_sign", "forget_dropped", "h_uses_old_c"])
def test_pins_catch_mutations(monkeypatch, kind):
    assert _all_pins_pass(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(orc, "lstm_cell", _mut_cell(kind))
    assert not _all_pins_pass(), f"mutation {kind} was not caught by any pin"


def test_pins_catch_layer_input_mistake(monkeypatch):
    """Feeding x (instead of the lower layer's h) to every layer must be caught."""
    real_layer = orc.lstm_layer

    def forward_wrong(x, W, R, b, h0=None, c0=None):
        L = len(W)
        x64 = np.asarray(x, dtype=np.float64)
        T, B, _ = x64.shape
        H = np.asarray(R[0]).shape[1]
        hT = np.empty((L, B, H))
        cT = np.empty((L, B, H))
        U = None
        for l in range(L):
            src = x64 if (l == 0 or x64.shape[2] == H) else U
            hl = np.zeros((B, H)) if h0 is None else np.asarray(h0[l], dtype=np.float64)
            cl = np.zeros((B, H)) if c0 is None else np.asarray(c0[l], dtype=np.float64)
            U, hT[l], cT[l] = real_layer(np.asarray(W[l], dtype=np.float64), np.asarray(R[l], dtype=np.float64),
                                         np.asarray(b[l], dtype=np.float64), src, hl, cl)
        return U, hT, cT

    assert _all_pins_pass()
    monkeypatch.setattr(orc, "lstm_forward", forward_wrong)
    # P4 at I == H so the wrong input has the right width
    err, bound = pins.check_p4(L=2, I=2, H=2, B=1, T=3)
    assert err > bound
