"""CPU tests of the C-ABI library: it loads, exports every declared entry
point, and its host-only logic (validation, workspace size, planner) behaves.
No compute call is made here (there may be no GPU)."""
import ctypes
import os
import re

import pytest

import lstm_inputs as li
import stacked_lstm_forward_amd as sl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header=None):
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h") or (header and fn != header):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, re.M):
            names.append(m.group(1))
    return names


def test_library_loads_and_exports_all_declared_symbols():
    lib = sl.load_library()
    names = declared_functions("lstm_fwd.h")
    assert set(names) == set(sl.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_peaks_library_loads_and_exports_all_declared_symbols():
    from stacked_lstm_forward_amd import peaks
    lib = peaks.load_library()
    names = declared_functions("lstm_peaks.h")
    assert set(names) == set(peaks.EXPORTED), names
    for n in names:
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value
    # host-only sizing (no GPU call)
    assert lib.lstm_peak_step_ws_bytes(256, 1, 1024, 10) == 256 + 256 * 128 + 10 * 256 * 1024
    assert lib.lstm_peak_step_ws_bytes(256, 8, 384, 10) == 256 + 256 * 128 + 10 * 32 * 384
    assert lib.lstm_peak_step_ws_bytes(256, 1, 24, 10) == 0      # slice not a multiple of 16
    assert lib.lstm_peak_step_ws_bytes(512, 1, 16, 10) == 0      # more than 256 active workgroups


def test_training_entry_points_exported():
    lib = sl.load_library()
    names = declared_functions("lstm_bwd.h")
    assert set(names) == set(sl.EXPORTED_TRAIN), names
    for n in names:
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_every_header_is_covered():
    assert set(declared_functions()) == set(declared_functions("lstm_fwd.h")) | set(
        declared_functions("lstm_peaks.h")) | set(declared_functions("lstm_bwd.h"))


def test_training_sizes_and_host_checks():
    d = sl.make_desc(2, 24, 16, 3, 5, "f32")
    tbh = 2 * 5 * 3 * 16
    assert sl.lstm_train_reserve_size(d) == (tbh * (16 + 4 + 4) + 255) // 256 * 256
    assert sl.lstm_bwd_workspace_size(d) > 0
    g = sl.make_desc(2, 24, 16, 3, 5, "f32", "gru")
    assert sl.lstm_train_reserve_size(g) == 0 and sl.lstm_bwd_workspace_size(g) == 0
    # refusals happen on the host, before any launch (no GPU needed); the 15
    # tensor arguments x .. db, then the workspace, then the stream
    args = [FAKE] * 15
    assert sl.lstm_bwd(g, *args, FAKE, 0) == sl.LSTM_ERR_UNSUPPORTED
    assert sl.lstm_bwd(None, *args, FAKE, 0) == sl.LSTM_ERR_INVALID_ARG
    assert sl.lstm_bwd(d, *args, FAKE + 16, 0) == sl.LSTM_ERR_WORKSPACE
    assert sl.lstm_bwd(d, *args, None, 0) == sl.LSTM_ERR_WORKSPACE
    missing = list(args)
    missing[5] = None  # reserve
    assert sl.lstm_bwd(d, *missing, FAKE, 0) == sl.LSTM_ERR_INVALID_ARG
    assert sl.lstm_fwd_train(d, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 0) == \
        sl.LSTM_ERR_INVALID_ARG


def test_one_hip_runtime_after_loading():
    """Loading the library before anything imported torch must still leave one
    HIP runtime in the process (torch's): two would make torch's streams and
    memory foreign to the library.  Checked in a fresh interpreter; loading
    touches no GPU."""
    import subprocess
    import sys
    code = ("import stacked_lstm_forward_amd as sl; sl.load_library(); import torch; "
            "maps = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def test_backward_chain_selection():
    """Which shapes run the backward's recurrent chain on chip (host rule, no GPU)."""
    on = lambda L, I, H, B, T, dt, cell="lstm": sl.lstm_bwd_chain_on_chip(  # noqa: E731
        sl.make_desc(L, I, H, B, T, dt, cell))
    # the instantiated (dtype, H): H / 16 workgroups, each a quarter of K
    for H in (128, 256, 512, 1024, 1536, 2048, 3072, 4096):
        assert on(1, 64, H, 16, 4, "bf16"), H
    for H in (128, 256, 512, 1024):
        assert on(1, 64, H, 16, 4, "f32"), H
    for H, dt in ((64, "bf16"), (192, "bf16"), (768, "bf16"), (2560, "bf16"), (96, "f32"), (2048, "f32"),
                  (4096, "f32"), (300, "bf16")):
        assert not on(1, 64, H, 16, 4, dt), (H, dt)
    # batch tiles: up to 4 (64 sequences; a third runs as a padded fourth), 2 at H = 4096
    assert on(1, 64, 256, 64, 4, "bf16") and on(1, 64, 256, 40, 4, "bf16") and not on(1, 64, 256, 65, 4, "bf16")
    assert on(1, 64, 4096, 32, 4, "bf16") and not on(1, 64, 4096, 33, 4, "bf16")
    # every workload
    assert on(4, 512, 512, 64, 100, "f32") and on(8, 256, 256, 64, 200, "bf16")
    assert on(4, 4096, 4096, 32, 50, "bf16") and on(1, 1536, 1536, 4, 2048, "bf16")
    assert on(1, 128, 128, 8, 16, "f32")
    # 32-bit offsets inside the kernel: T B 4H and the T + 1 exchange slots stay below 2^31
    assert on(1, 64, 4096, 32, 4094, "bf16") and not on(1, 64, 4096, 32, 4095, "bf16")
    # LSTM only; invalid descriptors are refused
    assert not on(1, 64, 256, 16, 4, "bf16", "gru")
    assert not sl.lstm_bwd_chain_on_chip(sl.make_desc(1, 64, 256, 0, 4, "bf16"))


def test_status_strings():
    assert sl.lstm_status_string(sl.LSTM_OK) == "LSTM_OK"
    assert sl.lstm_status_string(sl.LSTM_ERR_BARRIER_TIMEOUT) == "LSTM_ERR_BARRIER_TIMEOUT"
    assert sl.lstm_status_string(99) == "LSTM_ERR_UNKNOWN"


FAKE = 1 << 20  # a non-null, 256-aligned fake address; validation never dereferences it


def test_validate_error_paths():
    d = sl.make_desc(2, 8, 8, 3, 4, "f32")
    need = sl.lstm_fwd_workspace_size(d)
    assert need > 0
    v = sl.lstm_fwd_validate
    assert v(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need) == sl.LSTM_OK
    assert v(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need) == sl.LSTM_ERR_INVALID_ARG
    for k in range(5):  # each required tensor
        args = [FAKE] * 5
        args[k] = None
        assert v(d, *args, FAKE, need) == sl.LSTM_ERR_INVALID_ARG
    assert v(d, FAKE, FAKE, FAKE, FAKE, FAKE, None, need) == sl.LSTM_ERR_WORKSPACE
    assert v(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need) == sl.LSTM_ERR_WORKSPACE   # misaligned
    assert v(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1) == sl.LSTM_ERR_WORKSPACE
    for field in ("L", "I", "H", "B", "T"):
        bad = sl.make_desc(2, 8, 8, 3, 4, "f32")
        setattr(bad, field, 0)
        assert v(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need) == sl.LSTM_ERR_INVALID_ARG
        setattr(bad, field, -3)
        assert v(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need) == sl.LSTM_ERR_INVALID_ARG
    bad = sl.make_desc(2, 8, 8, 3, 4, 7)
    assert v(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need) == sl.LSTM_ERR_INVALID_ARG
    assert sl.lstm_fwd_workspace_size(bad) == 0


def test_unsupported_batch():
    d = sl.make_desc(1, 8, 8, 257, 4, "f32")
    assert sl.lstm_fwd_workspace_size(d) == 0
    assert sl.lstm_fwd_validate(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30) == sl.LSTM_ERR_UNSUPPORTED


def test_workspace_size_formula():
    for name, c in li.CONFIGS.items():
        d = sl.make_desc(c.L, c.I, c.H, c.B, c.T, c.dtype)
        n = sl.lstm_fwd_workspace_size(d)
        ds = 2 if c.dtype == "bf16" else 4
        mt = (c.H + 3) // 4
        kc = 64 if c.dtype == "bf16" else 32
        # an exchange slot holds h_t row-major ([B][H]) or in load order (16-column
        # tiles x 16 x KC chunks), whichever is larger, from a 256-byte boundary
        elems = max(c.B * c.H, -(-c.B // 16) * 16 * -(-c.H // kc) * kc)
        slot = -(-elems * ds // 256) * 256
        # L x T exchange slots, plus T + 1 slots of one layer's load-order
        # exchange (slot 0: h0 for the register-resident kernel)
        expect = 256 + c.L * 1024 * 128 + c.T * mt * c.B * 16 * 4 + c.L * c.T * slot + (c.T + 1) * slot
        assert expect <= n <= expect + 4 * 256, (name, n, expect)


EXPECTED_REGIME = {"c1": 1, "c2": 2, "c3": 2, "c4": 1, "c5": 1}


@pytest.mark.parametrize("name", sorted(li.CONFIGS))
def test_planner_on_mi355x_shape(name):
    c = li.CONFIGS[name]
    d = sl.make_desc(c.L, c.I, c.H, c.B, c.T, c.dtype)
    info = sl.lstm_fwd_plan(d, 0, 256, 160 * 1024)
    assert info.regime == EXPECTED_REGIME[name]
    assert info.grid <= 256 and info.grid % 8 == 0
    assert info.lds_bytes + 256 <= 160 * 1024
    mt = (c.H + 3) // 4
    for k in range(info.layers_per_launch):
        assert info.wg_per_layer[k] * info.mtiles_per_wg[k] >= mt
    if name in ("c2", "c3", "c5", "c1"):
        assert info.weights_on_chip
    if name == "c4":
        # 128 MiB of R per layer: 48 of each wave's 64 blocks in registers, the rest in LDS
        assert info.weights_on_chip and info.weight_blocks_in_registers == 48 and not info.weights_streamed
    else:
        assert info.weight_blocks_in_registers == 0
    if info.regime == 2:
        assert info.layers_per_launch == c.L
        assert info.num_launches == 2  # clear + one recurrent launch: every input product fused
        assert info.input_gemms == 0
        assert len(set(info.mtiles_per_wg[:c.L])) == 1  # equal tiles per workgroup in every layer
    else:
        assert info.num_launches == 2 * c.L


def test_planner_wavefront_falls_back_to_hoisted_first_layer():
    # [W_0 | R_0] rows of a 4096-wide input do not fit one workgroup's LDS
    info = sl.lstm_fwd_plan(sl.make_desc(2, 4096, 16, 4, 3, "f32"), 2, 256, 160 * 1024)
    assert info.regime == 2 and info.input_gemms == 1 and info.num_launches == 2
    info = sl.lstm_fwd_plan(sl.make_desc(2, 64, 16, 4, 3, "f32"), 2, 256, 160 * 1024)
    assert info.regime == 2 and info.input_gemms == 0


def test_planner_forced_regimes_and_small_devices():
    d = sl.make_desc(3, 5, 7, 3, 4, "bf16")
    for regime in (1, 2):
        info = sl.lstm_fwd_plan(d, regime, 256, 160 * 1024)
        assert info.regime == regime
    # a tiny device: everything still gets a partition with at least one M-tile per workgroup
    info = sl.lstm_fwd_plan(sl.make_desc(4, 64, 64, 16, 4, "f32"), 1, 8, 64 * 1024)
    assert info.grid <= 8
    with pytest.raises(sl.LstmError):
        sl.lstm_fwd_plan(sl.make_desc(1, 4, 4, 4, 4, "f32"), 9, 256, 160 * 1024)


def test_planner_data_valid_exchange_only_on_small_single_layer_grids():
    """Counter-free exchange: single hoisted layers with B < 16 and at most 64 workgroups."""
    expect = {"c1": True, "c2": False, "c3": False, "c4": False, "c5": False}
    for name, want in expect.items():
        c = li.CONFIGS[name]
        info = sl.lstm_fwd_plan(sl.make_desc(c.L, c.I, c.H, c.B, c.T, c.dtype), 0, 256, 160 * 1024)
        assert bool(info.data_valid_exchange) == want, name
    for (H, B, dt), want in {(256, 4, "bf16"): True, (256, 8, "f32"): True, (512, 4, "bf16"): False,
                             (128, 16, "bf16"): False, (128, 8, "f32"): True}.items():
        info = sl.lstm_fwd_plan(sl.make_desc(2, H, H, B, 10, dt), 1, 256, 160 * 1024)
        assert info.grid <= 64 or not want
        assert bool(info.data_valid_exchange) == want, (H, B, dt)
    # the wavefront never uses it
    info = sl.lstm_fwd_plan(sl.make_desc(2, 128, 128, 8, 10, "bf16"), 2, 256, 160 * 1024)
    assert not info.data_valid_exchange


def test_planner_keeps_four_chunks_per_wave_in_8_wave_launches():
    """8-wave launches take the widest K split that leaves every wave >= 4 chunks:
    the 8-layer bf16 H=256 stack (8 chunks per tile row) splits 2 ways, the 4-layer
    fp32 H=512 stack (32 chunks) 4 ways; 4-wave single-layer launches are unchanged."""
    want = {"c2": (4, [2, 2]), "c3": (2, [2, 1]), "c5": (4, [2, 1]), "c1": (4, [1, 1])}
    for name, (ks, tiles) in want.items():
        c = li.CONFIGS[name]
        info = sl.lstm_fwd_plan(sl.make_desc(c.L, c.I, c.H, c.B, c.T, c.dtype), 0, 256, 160 * 1024).as_dict()
        assert (info["ksplit"], info["wave_tiles"]) == (ks, tiles), name


def test_planner_refuses_past_the_limits():
    """B > 256 (16 column tiles) and L > 64 are refused before any launch."""
    for d in (sl.make_desc(2, 64, 64, 257, 3, "f32"), sl.make_desc(65, 32, 32, 4, 3, "bf16")):
        with pytest.raises(sl.LstmError) as ei:
            sl.lstm_fwd_plan(d, 0, 256, 160 * 1024)
        assert ei.value.status == sl.LSTM_ERR_UNSUPPORTED
    for d in (sl.make_desc(2, 64, 64, 256, 3, "f32"), sl.make_desc(64, 32, 32, 4, 3, "bf16")):
        assert sl.lstm_fwd_plan(d, 0, 256, 160 * 1024).grid > 0


def test_noalloc_host_checks_refuse_before_any_launch():
    """lstm_fwd_noalloc checks its arguments and the scratch limit on the host
    before any HIP call (so this runs without a GPU)."""
    d = sl.make_desc(4, 512, 512, 64, 100, "f32")  # needs 113 MiB, beyond the 64 MiB scratch
    assert sl.lstm_fwd_workspace_size(d) > sl.NOALLOC_MAX_WORKSPACE
    st = sl.lstm_fwd_noalloc(d, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, None, None, None, 0)
    assert st == sl.LSTM_ERR_WORKSPACE
    bad = sl.make_desc(0, 8, 8, 2, 2, "f32")
    assert sl.lstm_fwd_noalloc(bad, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, None, None, None, 0) == \
        sl.LSTM_ERR_INVALID_ARG
    small = sl.make_desc(1, 8, 8, 2, 2, "f32")
    assert sl.lstm_fwd_noalloc(small, None, None, None, FAKE, FAKE, FAKE, FAKE, None, None, None, 0) == \
        sl.LSTM_ERR_INVALID_ARG
