"""Host-side checks of libbt_ceilings (include/bt_ceilings.h) on a machine
without a GPU: it loads, exports what the header declares (and the binding
mirrors), and every argument error returns its status before any launch."""

import ctypes as C
import os
import re

from ternary_weight_decoder_bt_amd import ceilings as cl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bt_ceilings.h")
FAKE = 0x7F0000000000          # aligned, never dereferenced on the host


def header_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(btc_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = C.CDLL(cl.LIB_PATH)
    names = header_functions()
    assert "btc_mfma_i8_issue" in names and "btc_stream_read" in names
    assert not [n for n in names if not hasattr(L, n)]
    assert set(names) == set(cl.SIGNATURES)


def test_arguments_are_checked_before_launch():
    L = cl.lib()
    assert L.btc_mfma_i8_issue(1, 1, 1, 1, None, FAKE, None) == 1
    assert L.btc_mfma_i8_issue(1, 1, 1, 1, FAKE, None, None) == 1
    for blocks, iters in ((0, 1), (65537, 1), (1, 0), (1, (1 << 20) + 1)):
        assert L.btc_mfma_i8_issue(blocks, iters, 1, 1, FAKE, FAKE, None) == 2
    assert L.btc_stream_read(None, 16, 1, FAKE, None) == 1
    assert L.btc_stream_read(FAKE, 16, 1, None, None) == 1
    for ptr, nbytes, blocks, out in ((FAKE, 0, 1, FAKE), (FAKE, 24, 1, FAKE),
                                     (FAKE, (1 << 40) + 16, 1, FAKE), (FAKE, 16, 0, FAKE),
                                     (FAKE, 16, 65537, FAKE), (FAKE + 4, 16, 1, FAKE),
                                     (FAKE, 16, 1, FAKE + 8)):
        assert L.btc_stream_read(ptr, nbytes, blocks, out, None) == 2


def test_expected_issue_sum_wraps_like_int32():
    assert cl.expected_issue_sum(1, 1, 1) == 2048
    assert cl.expected_issue_sum(3, 5, -7) == 2048 * 3 * 5 * -7
    assert cl.expected_issue_sum(1 << 20, 1, 1) == -(1 << 31)     # 2^31 wraps
    assert cl.expected_issue_sum(1 << 21, 1, 1) == 0
