"""CPU pins of the oracle's GRU and simple-RNN cells (see tests/pins_cells.py)."""
import numpy as np
import pytest

import lstm_inputs as li
import oracle.lstm_oracle as orc
from tests import pins_cells as pc

NON_LSTM = ["gru", "rnn_tanh", "rnn_relu"]


@pytest.mark.parametrize("cell", NON_LSTM)
@pytest.mark.parametrize("shape", [dict(L=1, I=1, H=1, B=1, T=4), dict(L=2, I=3, H=4, B=3, T=5),
                                   dict(L=3, I=7, H=5, B=2, T=4, with_state=False)])
def test_q1_torch_float64(cell, shape):
    err, bound = pc.check_q1(cell, **shape)
    assert err <= bound, (cell, shape, err)


@pytest.mark.parametrize("cell", NON_LSTM)
def test_q1_torch_float64_on_stored_workload(cell):
    cfg = li.custom_config(2, 24, 16, 5, 6, "bf16", cfg_id=50, cell=cell)
    err, bound = pc.check_q1_inputs(li.make_inputs(cfg, random_state=True))
    assert err <= bound


@pytest.mark.parametrize("cell", NON_LSTM)
def test_q2_bruteforce(cell):
    err, bound = pc.check_q2(cell)
    assert err <= bound, err


def test_q3_gru_update_gate_open_carries_h_exactly():
    assert pc.check_q3_gru_update_gate_open()


def test_q3_gru_closed_gates_reduce_to_input_tanh():
    err, bound = pc.check_q3_gru_reset_and_update_closed()
    assert err <= bound


@pytest.mark.parametrize("cell", ["rnn_tanh", "rnn_relu"])
def test_q3_rnn_zero_recurrence(cell):
    err, bound, ok_sign = pc.check_q3_rnn_zero_recurrence(cell)
    assert err <= bound and ok_sign


@pytest.mark.parametrize("cell", NON_LSTM)
def test_q4_invariants(cell):
    assert pc.check_q4_layer_composition(cell)
    assert pc.check_q4_time_split(cell)


def test_lstm_entry_rejects_other_cells():
    cfg = li.custom_config(1, 2, 2, 1, 1, "f32", cell="gru")
    with pytest.raises(ValueError):
        orc.lstm_forward_inputs(li.make_inputs(cfg))


# ----------------------------------------------------------------------------- mutations
def _cells_pass(cell) -> bool:
    try:
        e1, b1 = pc.check_q1(cell, L=2, I=3, H=3, B=2, T=4)
        e2, b2 = pc.check_q2(cell, L=1, I=2, H=2, B=1, T=2)
        if e1 > b1 or e2 > b2:
            return False
        if cell == "gru":
            if not pc.check_q3_gru_update_gate_open():
                return False
            e3, b3 = pc.check_q3_gru_reset_and_update_closed()
            if e3 > b3:
                return False
        else:
            e3, b3, ok = pc.check_q3_rnn_zero_recurrence(cell)
            if e3 > b3 or not ok:
                return False
        return pc.check_q4_layer_composition(cell) and pc.check_q4_time_split(cell)
    except Exception:
        return False


def _mut_gru(kind):
    def cell(W, R, b, u, h):
        H = R.shape[1]
        Ru = R
        if kind == "transpose_R":
            Ru = R.reshape(3, H, H).transpose(0, 2, 1).reshape(3 * H, H)
        xu, rh = u @ W.T, h @ Ru.T
        r = orc.sigmoid(xu[:, :H] + rh[:, :H] + b[:H])
        z = orc.sigmoid(xu[:, H:2 * H] + rh[:, H:2 * H] + b[H:2 * H])
        if kind == "swap_rz":
            r, z = z, r
        nin, nh, bwn, brn = xu[:, 2 * H:], rh[:, 2 * H:], b[2 * H:3 * H], b[3 * H:]
        if kind == "reset_outside_bias":
            n = np.tanh(nin + bwn + r * nh + brn)
        elif kind == "reset_on_input":
            n = np.tanh(r * (nin + bwn) + nh + brn)
        elif kind == "no_reset":
            n = np.tanh(nin + bwn + nh + brn)
        else:
            n = np.tanh(nin + bwn + r * (nh + brn))
        if kind == "swap_interp":
            return z * n + (1.0 - z) * h
        return (1.0 - z) * n + z * h
    return cell


@pytest.mark.parametrize("kind", ["transpose_R", "swap_rz", "reset_outside_bias", "reset_on_input", "no_reset",
                                  "swap_interp"])
def test_gru_pins_catch_mutations(monkeypatch, kind):
    assert _cells_pass("gru"), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(orc, "gru_cell", _mut_gru(kind))
    assert not _cells_pass("gru"), f"GRU mutation {kind} was not caught"


def _mut_rnn(kind):
    def cell(W, R, b, u, h, relu):
        Ru = R.T if kind == "transpose_R" else R
        p = u @ W.T + h @ Ru.T + (0.0 if kind == "drop_bias" else b)
        if kind == "swap_act":
            relu = not relu
        return np.maximum(p, 0.0) if relu else np.tanh(p)
    return cell


@pytest.mark.parametrize("cell", ["rnn_tanh", "rnn_relu"])
@pytest.mark.parametrize("kind", ["transpose_R", "drop_bias", "swap_act"])
def test_rnn_pins_catch_mutations(monkeypatch, cell, kind):
    assert _cells_pass(cell)
    monkeypatch.setattr(orc, "rnn_cell", _mut_rnn(kind))
    assert not _cells_pass(cell), f"{cell} mutation {kind} was not caught"
