"""Python binding of the gfx950 stacked-LSTM forward library (``include/lstm_fwd.h``).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of ``lib/liblstm_fwd.so``.  PyTorch supplies device memory and streams.
If the library is not built, loading it raises; there is no fallback.

The functions carry the C names:

    lstm_fwd_workspace_size(desc) -> int
    lstm_fwd(desc, x, h0, c0, W, R, b, y, hT, cT, ws, stream=None) -> status
    lstm_fwd_ex(desc, ..., ws, stream=None, opts=None) -> status
    lstm_fwd_validate(desc, x, W, R, b, y, ws, ws_bytes) -> status
    lstm_fwd_last_error(ws, stream=None) -> status
    lstm_fwd_plan(desc, force_regime=0, num_cus=0, lds_per_cu=0) -> PlanInfo
    lstm_status_string(status) -> str
    lstm_fwd_noalloc(desc, x, h0, c0, W, R, b, y, hT, cT, dev_status=None, stream=None) -> status
    lstm_train_reserve_size(desc), lstm_bwd_workspace_size(desc) -> int
    lstm_bwd_chain_on_chip(desc) -> bool
    lstm_fwd_train(desc, x, h0, c0, W, R, b, y, hT, cT, reserve, ws, stream=None) -> status
    lstm_bwd(desc, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db, ws, stream=None) -> status
    lstm_fwd_train_ex(..., opts) / lstm_bwd_ex(..., opts): the same with LstmOpts / BwdOpts

Tensor arguments may be torch tensors (their ``data_ptr()``), raw integer
device addresses, or None for the nullable ones (h0, c0, hT, cT).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "liblstm_fwd.so")

LSTM_F32, LSTM_BF16 = 0, 1
LSTM_OK, LSTM_ERR_INVALID_ARG, LSTM_ERR_UNSUPPORTED, LSTM_ERR_WORKSPACE, LSTM_ERR_HIP, LSTM_ERR_BARRIER_TIMEOUT = range(6)
LSTM_REGIME_AUTO, LSTM_REGIME_LAYERWISE, LSTM_REGIME_WAVEFRONT = 0, 1, 2
LSTM_KERNEL_INPUT_GEMM, LSTM_KERNEL_RECURRENT, LSTM_KERNEL_CLEAR = 1, 2, 3
LSTM_CELL_LSTM, LSTM_CELL_GRU, LSTM_CELL_RNN_TANH, LSTM_CELL_RNN_RELU = range(4)
CELL_IDS = {"lstm": LSTM_CELL_LSTM, "gru": LSTM_CELL_GRU, "rnn_tanh": LSTM_CELL_RNN_TANH,
            "rnn_relu": LSTM_CELL_RNN_RELU}

EXPORTED = ("lstm_fwd_workspace_size", "lstm_fwd", "lstm_fwd_ex", "lstm_status_string",
            "lstm_fwd_validate", "lstm_fwd_last_error", "lstm_fwd_plan", "lstm_fwd_noalloc")
NOALLOC_MAX_WORKSPACE = 64 << 20  # LSTM_FWD_NOALLOC_MAX_WORKSPACE
EXPORTED_TRAIN = ("lstm_train_reserve_size", "lstm_fwd_train", "lstm_fwd_train_ex", "lstm_bwd_workspace_size",
                  "lstm_bwd_chain_on_chip", "lstm_bwd", "lstm_bwd_ex", "lstm_bwd_last_error")


class LstmDesc(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("I", ctypes.c_int32), ("H", ctypes.c_int32),
                ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("dtype", ctypes.c_int32), ("cell", ctypes.c_int32)]


class BwdOpts(ctypes.Structure):
    _fields_ = [("plain_launch", ctypes.c_int32), ("reserved0", ctypes.c_int32), ("wait_timeout_us", ctypes.c_int64),
                ("reserved", ctypes.c_int32 * 4)]


class LstmOpts(ctypes.Structure):
    _fields_ = [("force_regime", ctypes.c_int32), ("max_launches", ctypes.c_int32),
                ("ev_start", ctypes.POINTER(ctypes.c_void_p)), ("ev_stop", ctypes.POINTER(ctypes.c_void_p)),
                ("launch_kind", ctypes.POINTER(ctypes.c_int32)), ("num_launches", ctypes.POINTER(ctypes.c_int32)),
                ("wait_timeout_us", ctypes.c_int64), ("trace", ctypes.c_void_p),
                ("trace_wgs", ctypes.c_int32), ("trace_stride", ctypes.c_int32), ("plain_launch", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("regime", ctypes.c_int32), ("num_launches", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("block", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("ksplit", ctypes.c_int32),
                ("weights_on_chip", ctypes.c_int32), ("layers_per_launch", ctypes.c_int32),
                ("wg_per_layer", ctypes.c_int32 * 16), ("mtiles_per_wg", ctypes.c_int32 * 16),
                ("tile_groups_m", ctypes.c_int32), ("tile_groups_n", ctypes.c_int32),
                ("wave_tiles_m", ctypes.c_int32), ("wave_tiles_n", ctypes.c_int32),
                ("weights_streamed", ctypes.c_int32), ("input_gemms", ctypes.c_int32),
                ("weight_blocks_in_registers", ctypes.c_int32), ("data_valid_exchange", ctypes.c_int32)]

    def as_dict(self) -> dict:
        n = self.layers_per_launch
        return {"regime": {1: "layerwise", 2: "wavefront"}.get(self.regime, self.regime),
                "num_launches": self.num_launches, "grid": self.grid, "block": self.block,
                "lds_bytes": self.lds_bytes, "ksplit": self.ksplit, "weights_on_chip": bool(self.weights_on_chip),
                "layers_per_launch": n, "wg_per_layer": list(self.wg_per_layer[:n]),
                "mtiles_per_wg": list(self.mtiles_per_wg[:n]),
                "tile_groups": [self.tile_groups_m, self.tile_groups_n],
                "wave_tiles": [self.wave_tiles_m, self.wave_tiles_n],
                "weights_streamed": bool(self.weights_streamed), "input_gemms": self.input_gemms,
                "weight_blocks_in_registers": self.weight_blocks_in_registers,
                "data_valid_exchange": bool(self.data_valid_exchange)}


class LstmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {lstm_status_string(status)} ({status})")


_lib = None


def load_library() -> ctypes.CDLL:
    """Load lib/liblstm_fwd.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m stacked_lstm_forward_amd.build`")
    # torch first: it brings its own HIP runtime (soname libamdhip64.so.7),
    # which the library's dependency then resolves to.  Loaded the other way
    # round, the process would hold two HIP runtimes and torch's streams and
    # memory would be foreign to the library's.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pdesc = ctypes.POINTER(LstmDesc)
    lib.lstm_fwd_workspace_size.argtypes = [pdesc]
    lib.lstm_fwd_workspace_size.restype = sz
    lib.lstm_fwd.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lstm_fwd.restype = i32
    lib.lstm_fwd_ex.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(LstmOpts)]
    lib.lstm_fwd_ex.restype = i32
    lib.lstm_status_string.argtypes = [i32]
    lib.lstm_status_string.restype = ctypes.c_char_p
    lib.lstm_fwd_validate.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, sz]
    lib.lstm_fwd_validate.restype = i32
    lib.lstm_fwd_last_error.argtypes = [vp, vp]
    lib.lstm_fwd_last_error.restype = i32
    lib.lstm_fwd_plan.argtypes = [pdesc, i32, i32, i32, ctypes.POINTER(PlanInfo)]
    lib.lstm_fwd_plan.restype = i32
    lib.lstm_fwd_noalloc.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lstm_fwd_noalloc.restype = i32
    lib.lstm_train_reserve_size.argtypes = [pdesc]
    lib.lstm_train_reserve_size.restype = sz
    lib.lstm_bwd_workspace_size.argtypes = [pdesc]
    lib.lstm_bwd_workspace_size.restype = sz
    lib.lstm_bwd_chain_on_chip.argtypes = [pdesc]
    lib.lstm_bwd_chain_on_chip.restype = i32
    lib.lstm_bwd_last_error.argtypes = [vp, vp]
    lib.lstm_bwd_last_error.restype = i32
    lib.lstm_fwd_train.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lstm_fwd_train.restype = i32
    lib.lstm_bwd.argtypes = [pdesc] + [vp] * 17
    lib.lstm_bwd.restype = i32
    lib.lstm_fwd_train_ex.argtypes = [pdesc] + [vp] * 12 + [ctypes.POINTER(LstmOpts)]
    lib.lstm_fwd_train_ex.restype = i32
    lib.lstm_bwd_ex.argtypes = [pdesc] + [vp] * 17 + [ctypes.POINTER(BwdOpts)]
    lib.lstm_bwd_ex.restype = i32
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(L: int, I: int, H: int, B: int, T: int, dtype, cell="lstm") -> LstmDesc:
    dt = {"f32": LSTM_F32, "bf16": LSTM_BF16}.get(dtype, dtype)
    return LstmDesc(L, I, H, B, T, dt, CELL_IDS.get(cell, cell))


def lstm_status_string(status: int) -> str:
    return load_library().lstm_status_string(status).decode()


def lstm_fwd_workspace_size(desc: LstmDesc) -> int:
    return int(load_library().lstm_fwd_workspace_size(ctypes.byref(desc)))


def lstm_fwd(desc, x, h0, c0, W, R, b, y, hT, cT, ws, stream=None) -> int:
    return int(load_library().lstm_fwd(ctypes.byref(desc), _ptr(x), _ptr(h0), _ptr(c0), _ptr(W), _ptr(R), _ptr(b),
                                       _ptr(y), _ptr(hT), _ptr(cT), _ptr(ws), _stream(stream)))


def lstm_fwd_ex(desc, x, h0, c0, W, R, b, y, hT, cT, ws, stream=None, opts: Optional[LstmOpts] = None) -> int:
    return int(load_library().lstm_fwd_ex(ctypes.byref(desc), _ptr(x), _ptr(h0), _ptr(c0), _ptr(W), _ptr(R),
                                          _ptr(b), _ptr(y), _ptr(hT), _ptr(cT), _ptr(ws), _stream(stream),
                                          None if opts is None else ctypes.byref(opts)))


def lstm_fwd_noalloc(desc, x, h0, c0, W, R, b, y, hT, cT, dev_status=None, stream=None) -> int:
    return int(load_library().lstm_fwd_noalloc(None if desc is None else ctypes.byref(desc), _ptr(x), _ptr(h0),
                                               _ptr(c0), _ptr(W), _ptr(R), _ptr(b), _ptr(y), _ptr(hT), _ptr(cT),
                                               _ptr(dev_status), _stream(stream)))


def lstm_train_reserve_size(desc) -> int:
    return int(load_library().lstm_train_reserve_size(ctypes.byref(desc)))


def lstm_bwd_last_error(ws, stream=None) -> int:
    return int(load_library().lstm_bwd_last_error(_ptr(ws), _stream(stream)))


def lstm_bwd_workspace_size(desc) -> int:
    return int(load_library().lstm_bwd_workspace_size(ctypes.byref(desc)))


def lstm_bwd_chain_on_chip(desc) -> bool:
    return bool(load_library().lstm_bwd_chain_on_chip(ctypes.byref(desc)))


def lstm_fwd_train(desc, x, h0, c0, W, R, b, y, hT, cT, reserve, ws, stream=None) -> int:
    return int(load_library().lstm_fwd_train(ctypes.byref(desc), _ptr(x), _ptr(h0), _ptr(c0), _ptr(W), _ptr(R),
                                             _ptr(b), _ptr(y), _ptr(hT), _ptr(cT), _ptr(reserve), _ptr(ws),
                                             _stream(stream)))


def lstm_bwd(desc, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db, ws, stream=None) -> int:
    return int(load_library().lstm_bwd(None if desc is None else ctypes.byref(desc), _ptr(x), _ptr(h0), _ptr(c0),
                                       _ptr(W), _ptr(R), _ptr(reserve), _ptr(dy), _ptr(dhT), _ptr(dcT), _ptr(dx),
                                       _ptr(dh0), _ptr(dc0), _ptr(dW), _ptr(dR), _ptr(db), _ptr(ws),
                                       _stream(stream)))


def lstm_fwd_train_ex(desc, x, h0, c0, W, R, b, y, hT, cT, reserve, ws, stream=None, opts=None) -> int:
    return int(load_library().lstm_fwd_train_ex(ctypes.byref(desc), _ptr(x), _ptr(h0), _ptr(c0), _ptr(W), _ptr(R),
                                                _ptr(b), _ptr(y), _ptr(hT), _ptr(cT), _ptr(reserve), _ptr(ws),
                                                _stream(stream), None if opts is None else ctypes.byref(opts)))


def lstm_bwd_ex(desc, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db, ws, stream=None,
                opts=None) -> int:
    return int(load_library().lstm_bwd_ex(None if desc is None else ctypes.byref(desc), _ptr(x), _ptr(h0), _ptr(c0),
                                          _ptr(W), _ptr(R), _ptr(reserve), _ptr(dy), _ptr(dhT), _ptr(dcT), _ptr(dx),
                                          _ptr(dh0), _ptr(dc0), _ptr(dW), _ptr(dR), _ptr(db), _ptr(ws),
                                          _stream(stream), None if opts is None else ctypes.byref(opts)))


def lstm_fwd_validate(desc, x, W, R, b, y, ws, ws_bytes: int) -> int:
    return int(load_library().lstm_fwd_validate(None if desc is None else ctypes.byref(desc), _ptr(x), _ptr(W),
                                                _ptr(R), _ptr(b), _ptr(y), _ptr(ws), ws_bytes))


def lstm_fwd_last_error(ws, stream=None) -> int:
    return int(load_library().lstm_fwd_last_error(_ptr(ws), _stream(stream)))


def lstm_fwd_plan(desc, force_regime: int = 0, num_cus: int = 0, lds_per_cu: int = 0) -> PlanInfo:
    info = PlanInfo()
    st = load_library().lstm_fwd_plan(ctypes.byref(desc), force_regime, num_cus, lds_per_cu, ctypes.byref(info))
    if st != LSTM_OK:
        raise LstmError(st, "lstm_fwd_plan")
    return info


def check(status: int, what: str = "lstm_fwd") -> None:
    if status != LSTM_OK:
        raise LstmError(status, what)
