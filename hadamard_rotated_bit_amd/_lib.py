"""ctypes loader for libhq.so (argument marshalling only; no computation here)."""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhq.so")
HEADER = os.path.join(HERE, "..", "include", "hq.h")

DESC_FIELDS = ["d_in", "d_out", "block", "a_bits", "w_bits", "center", "smooth", "rank",
               "x_dtype", "w_dtype", "y_dtype", "gemm", "group"]


class HqDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in DESC_FIELDS]


class HqLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ["total", "w_codes", "w_scale", "c", "bias", "sigma_inv", "l1_hi", "l1_lo",
                 "l2_hi", "l2_lo", "weight"]] + [("d_out_pad", ctypes.c_int64)]


class HqIntDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ["d_in", "d_out", "block", "w_dtype", "side", "in_block", "act", "post_block"]]


class HqIntLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ["total", "w_codes", "w_scale", "b_int", "mult", "shift", "wbar"]] + [
        ("d_out_pad", ctypes.c_int64)] + [
        (n, ctypes.c_size_t) for n in ["lut", "mult_in", "shift_in"]]


HQ_CODES_I8, HQ_CODES_E2M3 = 0, 1
HQ_GEMM_AUTO, HQ_GEMM_I8 = 0, 1
HQ_CENTER_NONE, HQ_CENTER_TOKEN, HQ_CENTER_CHANNEL = 0, 1, 2
HQ_INT_WH, HQ_INT_DH = 0, 1
HQ_INT_ACT_NONE, HQ_INT_ACT_RELU, HQ_INT_ACT_SILU, HQ_INT_ACT_GELU = 0, 1, 2, 3

HQ_OK, HQ_ERR_INVALID_ARG, HQ_ERR_UNSUPPORTED, HQ_ERR_WORKSPACE, HQ_ERR_BAD_PREPARED, \
    HQ_ERR_HIP = 0, -1, -2, -3, -4, -5

_P = ctypes.c_void_p
_D = ctypes.POINTER(HqDesc)
_W = ctypes.POINTER(HqIntDesc)
_I64 = ctypes.c_int64
_SIGS = {
    "hq_abi_version": (ctypes.c_int, []),
    "hq_last_error": (ctypes.c_char_p, []),
    "hq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "hq_validate": (ctypes.c_int, [_D]),
    "hq_prepared_bytes": (ctypes.c_size_t, [_D]),
    "hq_prepared_layout_of": (ctypes.c_int, [_D, ctypes.POINTER(HqLayout)]),
    "hq_workspace_bytes": (ctypes.c_size_t, [_D, _I64]),
    "hq_code_format": (ctypes.c_int, [_D]),
    "hq_code_bytes": (ctypes.c_size_t, [_D, _I64]),
    "hq_channel_absmax": (ctypes.c_int, [_D, _P, _I64, _P, _P]),
    "hq_sigma": (ctypes.c_int, [_D, _P, _P, ctypes.c_float, _P, _P]),
    "hq_prepare_weights": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P]),
    "hq_check_prepared": (ctypes.c_int, [_D, _P, _P]),
    "hq_quant_linear": (ctypes.c_int, [_D, _P, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "hq_quant_linear_noalloc": (ctypes.c_int, [_D, _P, _P, _I64, _P, _P]),
    "hq_channel_center": (ctypes.c_int, [_D, _P, _P, _I64, _P, _P, _P, ctypes.c_size_t, _P]),
    "hq_act_quantize": (ctypes.c_int, [_D, _P, _P, _I64, _P, _P, _P, _P, _P]),
    "hq_act_quantize_ws": (ctypes.c_int, [_D, _P, _P, _I64, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "hq_act_transform": (ctypes.c_int, [_D, _P, _P, _I64, _P, _P, _P]),
    "hq_gemm_i32": (ctypes.c_int, [_D, _P, _P, _I64, _I64, _P, _P]),
    "hq_gemm_dequant": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _I64, _P, _P]),
    "hq_int_validate": (ctypes.c_int, [_W]),
    "hq_int_prepared_bytes": (ctypes.c_size_t, [_W]),
    "hq_int_prepared_layout_of": (ctypes.c_int, [_W, ctypes.POINTER(HqIntLayout)]),
    "hq_int_workspace_bytes": (ctypes.c_size_t, [_W, _I64]),
    "hq_int_prepare": (ctypes.c_int, [_W, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_float, _P, _P]),
    "hq_int_linear": (ctypes.c_int, [_W, _P, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "hq_int_requant": (ctypes.c_int, [_W, _P, _P, _I64, _P, _P]),
}

_lib = None


def header_functions() -> list:
    """Names of every function declared in include/hq.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hq_[a-z0-9_]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libhq.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                           "python -m hadamard_rotated_bit_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class HqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        self.status = status
        super().__init__(f"{load().hq_status_str(status).decode()}: {msg}")


def check(status: int) -> None:
    if status != HQ_OK:
        raise HqError(status, load().hq_last_error().decode())
