"""ctypes view of libbt_ceilings.so (include/bt_ceilings.h): the int8
matrix-core issue rate with the shader clock it ran at, and plain
streaming-read bandwidth, measured on the part the library runs on.

Not part of the matmul path. Loading fails loudly when the library has not
been built."""

from __future__ import annotations

import ctypes as C
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libbt_ceilings.so")

_p, _i32, _i64, _i8 = C.c_void_p, C.c_int, C.c_int64, C.c_int8

# name -> (restype, argtypes); mirrors include/bt_ceilings.h
SIGNATURES = {
    "btc_mfma_i8_issue": (_i32, [_i32, _i32, _i8, _i8, _p, _p, _p]),
    "btc_wall_clock_khz": (_i32, [_i32]),
    "btc_stream_read": (_i32, [_p, _i64, _i32, _p, _p]),
}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run the package's _build.py")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise RuntimeError(f"{what} failed with status {status}")


def mfma_i8_issue(blocks: int, iters: int, a_byte: int, b_byte: int, out, clocks,
                  stream: int = 0) -> None:
    """Launch the issue-rate kernel: out int32[blocks*256], clocks int64[4] (device)."""
    _check(lib().btc_mfma_i8_issue(blocks, iters, a_byte, b_byte, out.data_ptr(),
                                   clocks.data_ptr(), stream), "btc_mfma_i8_issue")


def expected_issue_sum(iters: int, a_byte: int, b_byte: int) -> int:
    """The value every thread of mfma_i8_issue writes, as a signed int32."""
    v = (32 * 64 * iters * a_byte * b_byte) & 0xFFFFFFFF
    return v - (1 << 32) if v >= 1 << 31 else v


def wall_clock_khz(device: int = 0) -> int:
    return lib().btc_wall_clock_khz(device)


def stream_read(ptr: int, nbytes: int, blocks: int, out, stream: int = 0) -> None:
    """Read nbytes at device address ptr; out uint32 as int32[blocks*16] (device)."""
    _check(lib().btc_stream_read(ptr, nbytes, blocks, out.data_ptr(), stream),
           "btc_stream_read")
