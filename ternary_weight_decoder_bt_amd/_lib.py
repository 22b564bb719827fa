"""ctypes view of libbt.so (the C ABI declared in include/bt.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""

from __future__ import annotations

import ctypes as C
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libbt.so")

BT_OK = 0
STATUS_NAMES = {0: "BT_OK", 1: "BT_ERR_NULL", 2: "BT_ERR_SHAPE", 3: "BT_ERR_VALUE",
                4: "BT_ERR_ALIGN", 5: "BT_ERR_DEVICE", 6: "BT_ERR_WORKSPACE"}

_i64, _i32, _sz, _p, _f = C.c_int64, C.c_int32, C.c_size_t, C.c_void_p, C.c_float

# name -> (restype, argtypes); mirrors include/bt.h
SIGNATURES = {
    "bt_status_string": (C.c_char_p, [C.c_int]),
    "bt_packed_bytes": (_sz, [_i64, _i64]),
    "bt_pack_ternary": (C.c_int, [_p, _i64, _i64, _p]),
    "bt_unpack_ternary": (C.c_int, [_p, _i64, _i64, _p]),
    "bt_ternarize_workspace_bytes": (_sz, [_i64, _i64]),
    "bt_ternarize": (C.c_int, [_p, _i64, _i64, _f, _p, _p, _p, _sz, _p]),
    "bt_ternarize_plan_bytes": (_sz, [_i32]),
    "bt_ternarize_plan_workspace_bytes": (_sz, [_p, _i32]),
    "bt_ternarize_plan_build": (C.c_int, [_p, _i32, _p, _sz, _p, _sz]),
    "bt_ternarize_grouped": (C.c_int, [_p, _p, _p]),
    "bt_repacked_bytes": (_sz, [_i64, _i64]),
    "bt_repack_ternary": (C.c_int, [_p, _i64, _i64, _p, _p]),
    "bt_quantize_act": (C.c_int, [_p, _i64, _i64, _p, _p, _p, _p]),
    "bt_rmsnorm_quantize": (C.c_int, [_p, _p, _f, _i64, _i64, _p, _p, _p, _p]),
    "bt_matmul_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bt_ternary_matmul": (C.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _f, _p, _p, _p, _sz, _p]),
    "bt_ternary_matmul_noalloc": (C.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _f, _p, _p, _p]),
    "bt_ternary_matmul_epilogue": (C.c_int, [_i64, _i64, _i64, _p, _p, _p, _p, _f, _p, _p, _p,
                                             _p, _sz, _p]),
    "bt_ternary_matmul_fused": (C.c_int, [_i64, _i64, _i64, _p, _p, _f, _p, _p, _p, _p, _p, _p,
                                          _sz, _p]),
    "bt_int8_repacked_bytes": (_sz, [_i64, _i64]),
    "bt_repack_int8": (C.c_int, [_p, _i64, _i64, _p, _p]),
    "bt_int8_matmul_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bt_int8_matmul": (C.c_int, [_i64, _i64, _i64, _p, _p, _p, _f, _p, _p, _p, _p, _sz, _p]),
    "bt_repack_plan_bytes": (_sz, [_i32]),
    "bt_repack_plan_build": (C.c_int, [_p, _i32, _p, _sz]),
    "bt_repack_ternary_grouped": (C.c_int, [_p, _p, _p]),
    "bt_quant_plan_bytes": (_sz, [_i32]),
    "bt_quant_plan_build": (C.c_int, [_p, _i32, _p, _sz]),
    "bt_quantize_act_grouped": (C.c_int, [_p, _p, _p]),
    "bt_matmul_plan_bytes": (_sz, [_i32]),
    "bt_matmul_plan_workspace_bytes": (_sz, [_p, _i32]),
    "bt_matmul_plan_build": (C.c_int, [_p, _i32, _p, _sz, _p, _sz]),
    "bt_ternary_matmul_grouped": (C.c_int, [_p, _p, _p]),
}


class BtEpilogue(C.Structure):
    _fields_ = [("bias", _p), ("layer_scale", _p), ("residual", _p), ("relu", _i32),
                ("reserved", _i32)]


class BtTernarizeDesc(C.Structure):
    _fields_ = [("w", _p), ("N", _i64), ("K", _i64), ("eps", _f), ("packed", _p), ("scale", _p)]


class BtRepackDesc(C.Structure):
    _fields_ = [("packed_dev", _p), ("wdev", _p), ("N", _i64), ("K", _i64)]


class BtQuantDesc(C.Structure):
    _fields_ = [("x", _p), ("xq", _p), ("xscale", _p), ("xsum", _p), ("M", _i64), ("K", _i64)]


class BtMatmulDesc(C.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("xq", _p), ("xscale", _p),
                ("xsum", _p), ("wdev", _p), ("w_scale", _f), ("y", _p), ("acc", _p), ("x", _p)]


class BtError(RuntimeError):
    """A bt_* call returned a status other than BT_OK."""

    def __init__(self, status: int, where: str = ""):
        self.status = status
        msg = STATUS_NAMES.get(status, str(status))
        try:
            msg += ": " + lib().bt_status_string(status).decode()
        except Exception:  # noqa: BLE001 - the message is best effort
            pass
        super().__init__(f"{where}: {msg}" if where else msg)


_LIB = None


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; build it with `python -c \"import __graft_entry__ as g; "
                "g.build()\"` (hipcc, gfx950). There is no fallback implementation.")
        # libbt.so needs libamdhip64.so.7, which torch also ships. Loading torch
        # first makes the library bind to the HIP runtime torch's streams and
        # memory come from; loaded the other way round, a process would carry two
        # runtimes and every launch on a torch stream would fail.
        import torch  # noqa: F401
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(status: int, where: str) -> None:
    if status != BT_OK:
        raise BtError(status, where)
