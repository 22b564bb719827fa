"""Host-side checks of libbt on a machine without a GPU.

The library loads and exports every function include/bt.h declares; the C++
canonical packing agrees byte for byte with the oracle; every error path
returns its documented status before anything is launched (so no call here
reaches the GPU).
"""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import ternary_weight_decoder_bt_amd as bt
from ternary_weight_decoder_bt_amd import _lib
from ternary_weight_decoder_bt_amd._lib import (BtEpilogue, BtMatmulDesc, BtQuantDesc, BtRepackDesc,
                                                 BtTernarizeDesc)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bt.h")

OK, NULL, SHAPE, VALUE, ALIGN, DEVICE, WORKSPACE = range(7)
FAKE = 0x7F0000000000          # an aligned address that is never dereferenced on the host


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bt_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for must in ("bt_pack_ternary", "bt_quantize_act", "bt_ternary_matmul", "bt_repack_ternary"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = C.CDLL(bt.LIB_PATH)
    missing = [n for n in header_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(header_functions()) == set(_lib.SIGNATURES)


def test_struct_layouts_match_header_sizes():
    # two int64 + pointer fields; no padding surprises between C and ctypes
    assert C.sizeof(BtQuantDesc) == 6 * 8
    assert C.sizeof(BtMatmulDesc) == 3 * 8 + 4 * 8 + 8 + 3 * 8
    assert C.sizeof(BtRepackDesc) == 4 * 8
    assert C.sizeof(BtEpilogue) == 3 * 8 + 2 * 4


def test_status_strings():
    L = bt.lib()
    for s in range(7):
        assert L.bt_status_string(s)
    assert b"unknown" in L.bt_status_string(99)


@pytest.mark.parametrize("n,k", [(1, 128), (3, 256), (40, 384), (17, 1536), (2, 8960)])
def test_pack_matches_oracle_bytes(n, k):
    w = np.random.default_rng(n * 1000 + k).integers(-1, 2, (n, k), dtype=np.int8)
    p = bt.pack_ternary(w)
    assert p.shape == (n, k // 4)
    assert np.array_equal(p, oracle.pack_ref(w))
    assert np.array_equal(bt.unpack_ternary(p, k), w)
    assert bt.packed_bytes(n, k) == oracle.packed_bytes(n, k) == p.nbytes


def test_pack_skewed_distributions():
    from synth import ternary_weights
    rng = np.random.default_rng(3)
    for p in [(0.3, 0.4, 0.3), (0.2, 0.6, 0.2), (1.0, 0.0, 0.0), (0.0, 0.0, 1.0)]:
        w = ternary_weights(rng, 32, 512, p)
        assert np.array_equal(bt.pack_ternary(w), oracle.pack_ref(w))


def test_pack_rejects_and_leaves_output_untouched():
    L = bt.lib()
    w = np.zeros((2, 128), np.int8)
    w[1, 77] = 2
    out = np.full((2, 32), 0xEE, np.uint8)
    assert L.bt_pack_ternary(w.ctypes.data, 2, 128, out.ctypes.data) == VALUE
    assert (out == 0xEE).all()
    assert L.bt_pack_ternary(None, 2, 128, out.ctypes.data) == NULL
    assert L.bt_pack_ternary(w.ctypes.data, 2, 100, out.ctypes.data) == SHAPE
    assert L.bt_pack_ternary(w.ctypes.data, 0, 128, out.ctypes.data) == SHAPE
    with pytest.raises(bt.BtError):
        bt.pack_ternary(w)


def test_unpack_rejects_code_three():
    p = np.full((1, 32), 0x55, np.uint8)
    p[0, 9] = 0xD5           # top pair = 0b11
    with pytest.raises(bt.BtError) as e:
        bt.unpack_ternary(p, 128)
    assert e.value.status == VALUE


def L_i8_ws(m, n, k):
    return bt.lib().bt_int8_matmul_workspace_bytes(m, n, k)


def test_sizes():
    assert bt.packed_bytes(1536, 1536) == 589_824
    assert bt.packed_bytes(10, 100) == 0 and bt.repacked_bytes(0, 128) == 0
    assert bt.repacked_bytes(40, 384) == 48 * 512 // 4     # rows to 16, K to 256
    assert bt.repacked_bytes(1536, 8960) == 1536 * 8960 // 4
    # the decode step's packed weights: 28 layers of the four projections
    total = 28 * sum(bt.packed_bytes(n, k) for k, n in
                     [(1536, 2048), (1536, 1536), (1536, 17920), (8960, 1536)])
    assert total == 327_548_928
    # GEMM: none when the output has enough tiles; split K (one M x N int32
    # slice of partial sums per K range) when it has fewer tiles than compute
    # units and a long K
    assert bt.matmul_workspace_bytes(4096, 17920, 1536) == 0
    assert bt.matmul_workspace_bytes(4096, 1536, 8960) == 0   # 512 tiles of 128 x 96
    assert bt.matmul_workspace_bytes(2048, 1536, 8960) == 0   # 256 tiles: one per CU
    assert bt.matmul_workspace_bytes(17, 1536, 1536) == 0     # too short a K to split
    # 3 x 24 tiles of 64 x 64, 35 stages: max(2, ceil(192/72)) = 3 ranges of 12
    assert bt.matmul_workspace_bytes(150, 1536, 8960) == 3 * 150 * 1536 * 4
    # 4 x 24 tiles of 64 x 64 at M = 512 ... 8 x 24: 2 ranges
    assert bt.matmul_workspace_bytes(512, 1536, 8960) == 2 * 512 * 1536 * 4
    # 12 x 16 tiles of 128 x 96: 2 ranges
    assert bt.matmul_workspace_bytes(1536, 1536, 8960) == 2 * 1536 * 1536 * 4
    # 14 x 15 tiles of 128 x 128 with K = 2560: the slices would cost more than the split gains
    assert bt.matmul_workspace_bytes(1700, 1900, 2560) == 0
    # int8: 3 x 32 tiles of 64 x 64, 64 stages of 128: ranges of at most 16 stages -> 4
    assert L_i8_ws(150, 2048, 8192) == 4 * 150 * 2048 * 4
    # a 6000 x 512 output over K = 2048: the slices would cost more than the split gains
    assert L_i8_ws(6000, 512, 2048) == 0
    # int8 weights of at most 64 KB with K <= 512 are held in LDS: never split
    assert L_i8_ws(480000, 128, 32) == 0 and L_i8_ws(30, 512, 128) == 0
    # GEMV: K is split only where M x K activations exceed one LDS slice
    assert bt.matmul_workspace_bytes(1, 1536, 1536) == 0
    assert bt.matmul_workspace_bytes(1, 1536, 8960) == 0
    # 16 x 8960 int8 rows: chunks of 9 steps -> 4 chunks; slices + scales/row sums
    assert bt.matmul_workspace_bytes(16, 1536, 8960) == 4 * 16 * 1536 * 4 + 256


def test_device_entry_points_validate_before_launch():
    L = bt.lib()
    f = FAKE
    # repack
    assert L.bt_repack_ternary(None, 16, 128, f, None) == NULL
    assert L.bt_repack_ternary(f, 16, 100, f, None) == SHAPE
    assert L.bt_repack_ternary(f + 4, 16, 128, f, None) == ALIGN
    # offline ternarization: w, packed, scale, workspace must be distinct buffers
    G = 1 << 30
    tz = lambda **kw: [kw.get("w", f), kw.get("N", 16), kw.get("K", 128), kw.get("eps", 0.0),
                       kw.get("p", f + G), kw.get("s", f + 2 * G), kw.get("ws", f + 3 * G),
                       kw.get("wsb", 256), None]
    assert L.bt_ternarize_workspace_bytes(16, 128) == 256
    assert L.bt_ternarize_workspace_bytes(1536, 1536) == 288 * 8 + 0  # 288 partials
    assert L.bt_ternarize_workspace_bytes(17920, 1536) == 1024 * 8
    assert L.bt_ternarize_workspace_bytes(16, 100) == 0
    assert L.bt_ternarize(*tz(w=None)) == NULL
    assert L.bt_ternarize(*tz(s=None)) == NULL
    assert L.bt_ternarize(*tz(K=100)) == SHAPE
    assert L.bt_ternarize(*tz(N=0)) == SHAPE
    assert L.bt_ternarize(*tz(eps=-1.0)) == VALUE
    assert L.bt_ternarize(*tz(eps=float("nan"))) == VALUE
    assert L.bt_ternarize(*tz(p=f + G + 4)) == ALIGN
    assert L.bt_ternarize(*tz(ws=None)) == WORKSPACE
    assert L.bt_ternarize(*tz(wsb=255)) == WORKSPACE
    assert L.bt_ternarize(*tz(p=f + 16 * 128)) == VALUE       # packed inside w (16x128 fp32)
    assert L.bt_ternarize(*tz(s=f + G + 256)) == VALUE        # scale inside packed (512 B)
    assert L.bt_ternarize(*tz(ws=f + G + 496)) == VALUE       # workspace overlaps packed
    # quantize
    assert L.bt_quantize_act(None, 1, 128, f, f, f, None) == NULL
    assert L.bt_quantize_act(f, 0, 128, f, f, f, None) == SHAPE
    assert L.bt_quantize_act(f, 1, 0, f, f, f, None) == SHAPE
    assert L.bt_quantize_act(f, 1, 128, f + 1, f, f, None) == ALIGN
    # I8_S
    assert L.bt_int8_repacked_bytes(16, 32) == 16 * 256
    assert L.bt_int8_repacked_bytes(17, 288) == 32 * 512
    for bad in ((0, 32), (16, 16), (16, 48), (16, 131072 + 32)):
        assert L.bt_int8_repacked_bytes(*bad) == 0
    assert L.bt_repack_int8(None, 16, 32, f, None) == NULL
    assert L.bt_repack_int8(f, 16, 48, f, None) == SHAPE
    assert L.bt_repack_int8(f, 16, 32, f + 8, None) == ALIGN
    i8 = lambda **kw: [kw.get("M", 2), kw.get("N", 16), kw.get("K", 64), kw.get("xq", f),
                       kw.get("xs", f), kw.get("w", f), kw.get("scale", 0.5), kw.get("epi", None),
                       kw.get("y", f), kw.get("acc", None), kw.get("ws", None),
                       kw.get("wsb", 0), None]
    assert L.bt_int8_matmul(*i8(w=None)) == NULL
    assert L.bt_int8_matmul(*i8(K=100)) == SHAPE
    assert L.bt_int8_matmul(*i8(M=0)) == SHAPE
    assert L.bt_int8_matmul(*i8(xs=f + 4)) == ALIGN
    assert L.bt_int8_matmul(*i8(scale=float("inf"))) == VALUE
    assert L.bt_int8_matmul(*i8(epi=C.byref(BtEpilogue(f + 4, None, None, 0, 0)))) == ALIGN
    need = L.bt_int8_matmul_workspace_bytes(150, 2048, 8192)
    assert L.bt_int8_matmul(*i8(M=150, N=2048, K=8192)) == WORKSPACE
    assert L.bt_int8_matmul(*i8(M=150, N=2048, K=8192, ws=f, wsb=need - 1)) == WORKSPACE
    assert L.bt_int8_matmul(*i8(M=150, N=2048, K=8192, ws=f + 4, wsb=need)) == ALIGN
    # RMS normalization + quantize
    assert L.bt_rmsnorm_quantize(f, None, 1e-6, 1, 128, f, f, f, None) == NULL
    assert L.bt_rmsnorm_quantize(f, f, 1e-6, 0, 128, f, f, f, None) == SHAPE
    assert L.bt_rmsnorm_quantize(f, f + 4, 1e-6, 1, 128, f, f, f, None) == ALIGN
    assert L.bt_rmsnorm_quantize(f, f, -1.0, 1, 128, f, f, f, None) == VALUE
    assert L.bt_rmsnorm_quantize(f, f, float("nan"), 1, 128, f, f, f, None) == VALUE
    assert L.bt_rmsnorm_quantize(f, f, float("inf"), 1, 128, f, f, f, None) == VALUE
    # matmul
    args = lambda **kw: [kw.get("M", 1), kw.get("N", 16), kw.get("K", 128), kw.get("xq", f),
                         kw.get("xs", f), kw.get("xsum", f), kw.get("w", f),
                         kw.get("scale", 0.5), kw.get("y", f), kw.get("acc", None),
                         kw.get("ws", None), kw.get("wsb", 0), None]
    assert L.bt_ternary_matmul(*args(xsum=None)) == NULL
    assert L.bt_ternary_matmul(*args(y=None)) == NULL
    assert L.bt_ternary_matmul(*args(K=130)) == SHAPE
    assert L.bt_ternary_matmul(*args(M=0)) == SHAPE
    assert L.bt_ternary_matmul(*args(w=f + 8)) == ALIGN
    assert L.bt_ternary_matmul(*args(acc=f + 2)) == ALIGN
    assert L.bt_ternary_matmul(*args(scale=float("inf"))) == VALUE
    assert L.bt_ternary_matmul(*args(scale=float("nan"))) == VALUE
    # a GEMM with a split K without (enough) workspace
    need = bt.matmul_workspace_bytes(150, 1536, 8960)
    assert L.bt_ternary_matmul(*args(M=150, N=1536, K=8960)) == WORKSPACE
    assert L.bt_ternary_matmul(*args(M=150, N=1536, K=8960, ws=f, wsb=need - 4)) == WORKSPACE
    assert L.bt_ternary_matmul(*args(M=150, N=1536, K=8960, ws=f + 4, wsb=need)) == ALIGN
    # the epilogue entry point: same checks, plus the epilogue's own
    eargs = lambda epi, **kw: args(**kw)[:8] + [epi] + args(**kw)[8:]
    assert L.bt_ternary_matmul_epilogue(*eargs(None, y=None)) == NULL
    assert L.bt_ternary_matmul_epilogue(*eargs(C.byref(BtEpilogue(f + 4, None, None, 0, 0)))) == ALIGN
    assert L.bt_ternary_matmul_epilogue(*eargs(C.byref(BtEpilogue(None, f + 8, None, 1, 0)))) == ALIGN
    # a residual that partly overlaps the output is refused; the output itself is fine
    assert L.bt_ternary_matmul_epilogue(*eargs(C.byref(BtEpilogue(None, None, f + 16, 0, 0)),
                                               M=2, N=16)) == VALUE
    assert L.bt_ternary_matmul_epilogue(*eargs(C.byref(BtEpilogue(None, None, f, 0, 0)),
                                               scale=float("nan"))) == VALUE
    # a split-K GEMV without (enough) workspace
    need = bt.matmul_workspace_bytes(16, 1536, 8960)
    assert L.bt_ternary_matmul(*args(M=16, N=1536, K=8960)) == WORKSPACE
    assert L.bt_ternary_matmul(*args(M=16, N=1536, K=8960, ws=f, wsb=need - 1)) == WORKSPACE
    assert L.bt_ternary_matmul(*args(M=16, N=1536, K=8960, ws=f + 4, wsb=need)) == ALIGN
    # fused quantize + GEMV: x, wdev, y required; q outputs optional; M <= 16
    fa = lambda **kw: [kw.get("M", 1), kw.get("N", 16), kw.get("K", 128), kw.get("x", f),
                       kw.get("w", f), kw.get("scale", 0.5), kw.get("y", f), None,
                       kw.get("xq", None), None, None, kw.get("ws", None), kw.get("wsb", 0), None]
    assert L.bt_ternary_matmul_fused(*fa(x=None)) == NULL
    assert L.bt_ternary_matmul_fused(*fa(M=17)) == SHAPE
    assert L.bt_ternary_matmul_fused(*fa(xq=f + 1)) == ALIGN
    assert L.bt_ternary_matmul_fused(*fa(scale=float("inf"))) == VALUE
    assert L.bt_ternary_matmul_fused(*fa(M=16, N=1536, K=8960)) == WORKSPACE


def test_k_bound_of_the_ternary_path():
    """K is capped at BT_MAX_K = 131072: |acc| <= 127 K stays below 2^24 (exact in
    int32 and in fp32), and the kernels' 32-bit offsets over 128 token rows of K
    bytes cannot wrap. Beyond it every size query is 0 and every call BT_ERR_SHAPE."""
    L = bt.lib()
    f = FAKE
    kmax = 131072
    assert 127 * kmax < 2 ** 24
    assert 128 * (kmax + 128) < 2 ** 31
    assert L.bt_packed_bytes(16, kmax) == 16 * kmax // 4
    assert L.bt_repacked_bytes(16, kmax) == 16 * kmax // 4
    for k in (kmax + 128, 1 << 24, 1 << 30):
        assert L.bt_packed_bytes(16, k) == 0
        assert L.bt_repacked_bytes(16, k) == 0
        assert L.bt_matmul_workspace_bytes(1, 16, k) == 0
        assert L.bt_matmul_workspace_bytes(4096, 16, k) == 0
        assert L.bt_repack_ternary(f, 16, k, f, None) == SHAPE
        for m in (1, 16, 17, 4096):
            assert L.bt_ternary_matmul(m, 16, k, f, f, f, f, 0.5, f, None, f, 1 << 40,
                                       None) == SHAPE
            assert L.bt_ternary_matmul_epilogue(m, 16, k, f, f, f, f, 0.5, None, f, None, f,
                                                1 << 40, None) == SHAPE
        assert L.bt_ternary_matmul_fused(1, 16, k, f, f, 0.5, f, None, None, None, None, f,
                                         1 << 40, None) == SHAPE
        d = (BtMatmulDesc * 1)(BtMatmulDesc(1, 16, k, f, f, f, f, 0.5, f, None, None))
        host = np.zeros(L.bt_matmul_plan_bytes(1), np.uint8)
        assert L.bt_matmul_plan_build(d, 1, None, 0, host.ctypes.data, host.nbytes) == SHAPE
        r = (BtRepackDesc * 1)(BtRepackDesc(f, f, 16, k))
        host = np.zeros(L.bt_repack_plan_bytes(1), np.uint8)
        assert L.bt_repack_plan_build(r, 1, host.ctypes.data, host.nbytes) == SHAPE
    # the host format follows the same bound
    w = np.zeros((1, kmax + 128), np.int8)
    out = np.zeros((kmax + 128) // 4, np.uint8)
    assert L.bt_pack_ternary(w.ctypes.data, 1, kmax + 128, out.ctypes.data) == SHAPE


def test_noalloc_entry_point_validates_before_launch():
    """bt_ternary_matmul_noalloc: bt_ternary_matmul's checks, and BT_ERR_WORKSPACE for a
    shape whose split-K partial sums would not fit the library's 16 MiB array (all
    returned before any runtime call, so they run without a GPU)."""
    L = bt.lib()
    f = FAKE
    na = lambda **kw: [kw.get("M", 1), kw.get("N", 16), kw.get("K", 128), kw.get("xq", f),
                       kw.get("xs", f), kw.get("xsum", f), kw.get("w", f),
                       kw.get("scale", 0.5), kw.get("y", f), kw.get("acc", None), None]
    assert L.bt_ternary_matmul_noalloc(*na(xq=None)) == NULL
    assert L.bt_ternary_matmul_noalloc(*na(xsum=None)) == NULL
    assert L.bt_ternary_matmul_noalloc(*na(y=None)) == NULL
    assert L.bt_ternary_matmul_noalloc(*na(K=130)) == SHAPE
    assert L.bt_ternary_matmul_noalloc(*na(K=131072 + 128)) == SHAPE
    assert L.bt_ternary_matmul_noalloc(*na(M=0)) == SHAPE
    assert L.bt_ternary_matmul_noalloc(*na(w=f + 8)) == ALIGN
    assert L.bt_ternary_matmul_noalloc(*na(acc=f + 4)) == ALIGN
    assert L.bt_ternary_matmul_noalloc(*na(scale=float("nan"))) == VALUE
    limit = 16 << 20
    assert bt.matmul_workspace_bytes(2054, 1024, 8960) > limit
    assert L.bt_ternary_matmul_noalloc(*na(M=2054, N=1024, K=8960)) == WORKSPACE
    # the decoder's split shapes fit
    for m, n, k in ((16, 1536, 8960), (512, 1536, 8960), (150, 1536, 8960)):
        assert 0 < bt.matmul_workspace_bytes(m, n, k) <= limit


def test_plan_building_on_host():
    L = bt.lib()
    f = FAKE
    q = (BtQuantDesc * 2)(BtQuantDesc(f, f, f, f, 3, 1536), BtQuantDesc(f, f, f, f, 1, 8960))
    nb = L.bt_quant_plan_bytes(2)
    host = np.zeros(nb, np.uint8)
    assert L.bt_quant_plan_build(q, 2, host.ctypes.data, nb) == OK
    hdr = host[:16].view(np.int64)
    assert hdr[1] == 2          # workgroups: 3 short rows (one per wave) + 1 long row
    assert L.bt_quant_plan_build(q, 2, host.ctypes.data, nb - 1) == WORKSPACE
    q[1].xsum = None
    assert L.bt_quant_plan_build(q, 2, host.ctypes.data, nb) == NULL
    # a grid beyond 2^31 - 1 workgroups is refused before the plan is written
    big = (BtQuantDesc * 2)(BtQuantDesc(f, f, f, f, 1 << 31, 8960),
                            BtQuantDesc(f, f, f, f, 1 << 31, 8960))
    host[:] = 0xAB
    assert L.bt_quant_plan_build(big, 2, host.ctypes.data, nb) == SHAPE
    assert (host == 0xAB).all()
    big[1].M = 1            # 2^31 + 1 workgroups: still too many
    assert L.bt_quant_plan_build(big, 2, host.ctypes.data, nb) == SHAPE
    assert (host == 0xAB).all()
    big[0].M = (1 << 31) - 2
    assert L.bt_quant_plan_build(big, 2, host.ctypes.data, nb) == OK
    assert host[:16].view(np.int64)[1] == (1 << 31) - 1

    m = (BtMatmulDesc * 2)(BtMatmulDesc(1, 2048, 1536, f, f, f, f, 0.02, f, None),
                           BtMatmulDesc(3, 1536, 8960, f, f, f, f, 0.03, f, f))
    nb = L.bt_matmul_plan_bytes(2)
    host = np.zeros(nb, np.uint8)
    assert L.bt_matmul_plan_workspace_bytes(m, 2) == 0      # both fit one LDS slice
    assert L.bt_matmul_plan_build(m, 2, None, 0, host.ctypes.data, nb) == OK
    # two tiles per wave, four waves per workgroup: 64 output rows per workgroup
    assert host[:16].view(np.int64)[1] == 2048 // 128 + 1536 // 128
    m[0].M = 17
    assert L.bt_matmul_plan_build(m, 2, None, 0, host.ctypes.data, nb) == SHAPE
    m[0].M = 1
    m[1].w_scale = float("nan")
    assert L.bt_matmul_plan_build(m, 2, None, 0, host.ctypes.data, nb) == VALUE
    m[1].w_scale = 0.5
    m[1].M = 16                     # 17 rows of 8960 int8 exceed the LDS slice: K is split
    need = L.bt_matmul_plan_workspace_bytes(m, 2)
    assert need > 0
    assert L.bt_matmul_plan_build(m, 2, None, 0, host.ctypes.data, nb) == WORKSPACE
    assert L.bt_matmul_plan_build(m, 2, f, need, host.ctypes.data, nb) == OK
    # a plan fuses quantization for all its projections or for none
    m[0].x = f
    assert L.bt_matmul_plan_build(m, 2, f, need, host.ctypes.data, nb) == VALUE
    m[1].x = f
    m[0].xq = m[0].xscale = m[0].xsum = None        # optional outputs when fused
    assert L.bt_matmul_plan_build(m, 2, f, need, host.ctypes.data, nb) == OK
    # the longest workgroups (K = 8960) are placed first in the grid
    assert host[:4].view(np.uint32)[0] == 0x42544646      # a fused plan
    # GemvDesc: 9 pointers, w_scale, then M, N, K as int32 (K at byte 84)
    first_k = host[16 + 84:16 + 88].view(np.int32)[0]
    assert first_k == 8960
    # a launch with a plan of the wrong kind is refused on the host
    assert L.bt_quantize_act_grouped(host.ctypes.data, f, None) == VALUE


def test_gemm_plan_building_on_host():
    """Descriptors with M > 16 build a grouped GEMM plan: quantized inputs only,
    no workspace, every descriptor on the same side of BT_GEMV_MAX_M; each
    projection gets min(64, its tiles per XCD) workgroup slots per XCD, and the
    projections are ordered by K, the longest first (stable)."""
    L = bt.lib()
    f = FAKE
    # one decoder layer at M=4096: qkv, o, gate_up (K=1536) and down (K=8960)
    shapes = [(2048, 1536), (1536, 1536), (17920, 1536), (1536, 8960)]
    m = (BtMatmulDesc * 4)(*[BtMatmulDesc(4096, n, k, f, f, f, f, 0.02, f, None, None)
                             for n, k in shapes])
    nb = L.bt_matmul_plan_bytes(4)
    host = np.zeros(nb, np.uint8)
    assert L.bt_matmul_plan_workspace_bytes(m, 4) == 0
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == OK
    assert host[:4].view(np.uint32)[0] == 0x42544D4D          # a GEMM plan
    tiles = [32 * -(-n // 256) for n, _ in shapes]             # 128 x 256 output tiles
    slots = host[8:16].view(np.int64)[0]                        # slots per XCD in the grid
    assert slots == sum(min(64, -(-t // 8)) for t in tiles) == 32 + 24 + 64 + 24
    # GemmArgs: 6 pointers, w_scale, then M, N, K (K at byte 60); K=8960 comes first,
    # the K=1536 projections keep their order (N at byte 56)
    ks = [host[16 + 152 * i + 60:16 + 152 * i + 64].view(np.int32)[0] for i in range(4)]
    ns = [host[16 + 152 * i + 56:16 + 152 * i + 60].view(np.int32)[0] for i in range(4)]
    assert ks == [8960, 1536, 1536, 1536]
    assert ns == [1536, 2048, 1536, 17920]
    # a launch with a GEMM plan is refused by the quantize launcher
    assert L.bt_quantize_act_grouped(host.ctypes.data, f, None) == VALUE
    # mixing GEMV (M <= 16) and GEMM projections, fused inputs, missing inputs
    m[1].M = 16
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == SHAPE
    m[1].M = 4096
    m[2].x = f
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == VALUE
    m[2].x = None
    m[3].xsum = None
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == NULL
    m[3].xsum = f
    m[3].y = f + 4
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == ALIGN
    m[3].y = f
    m[0].K = 131072 + 128
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == SHAPE
    # more output tiles than the kernel's int32 indexes hold; the plan is left unwritten
    m[0].K, m[0].M, m[0].N = 1536, (1 << 31) - 1, 1 << 30
    host[:] = 0
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == SHAPE
    assert not host.any()


def test_gemm_plan_split_k_on_host():
    """A projection of a GEMM plan with fewer 128 x 256 tiles than a quarter of
    the 512 resident slots and at least 32 stages of 128 along K is split into
    ranges of at most about 16 stages (even): one layer at M=512 has down (24
    tiles, 70 stages) in 5 ranges of 14, each range on its own 3 slots per XCD; the plan's
    workspace holds one M x N int32 slice per range and M zeros."""
    L = bt.lib()
    f = FAKE
    shapes = [(2048, 1536), (1536, 1536), (17920, 1536), (1536, 8960)]
    m = (BtMatmulDesc * 4)(*[BtMatmulDesc(512, n, k, f, f, f, f, 0.02, f, None, None)
                             for n, k in shapes])
    nb = L.bt_matmul_plan_bytes(4)
    host = np.zeros(nb, np.uint8)
    slice_bytes = (512 * 1536 * 4 + 255) // 256 * 256
    need = 5 * slice_bytes + 2048
    assert L.bt_matmul_plan_workspace_bytes(m, 4) == need
    assert L.bt_matmul_plan_build(m, 4, None, 0, host.ctypes.data, nb) == WORKSPACE
    assert L.bt_matmul_plan_build(m, 4, f, need - 1, host.ctypes.data, nb) == WORKSPACE
    assert L.bt_matmul_plan_build(m, 4, f + 8, need, host.ctypes.data, nb) == ALIGN
    assert L.bt_matmul_plan_build(m, 4, f, need, host.ctypes.data, nb) == OK
    slots = host[8:16].view(np.int64)[0]
    assert slots == 4 + 3 + 35 + 5 * 3
    # the unsplit shapes of the long prefill need no workspace (test above); nor does
    # a long K with many tiles, or a short K with few
    one = (BtMatmulDesc * 1)(BtMatmulDesc(4096, 1536, 8960, f, f, f, f, 0.02, f, None, None))
    assert L.bt_matmul_plan_workspace_bytes(one, 1) == 0
    one[0] = BtMatmulDesc(512, 1536, 3968, f, f, f, f, 0.02, f, None, None)   # 31 stages
    assert L.bt_matmul_plan_workspace_bytes(one, 1) == 0
    # 33 stages, one tile: ranges of 12, 12 and 9 stages
    one[0] = BtMatmulDesc(17, 40, 4224, f, f, f, f, 0.02, f, None, None)
    assert L.bt_matmul_plan_workspace_bytes(one, 1) == 3 * 2816 + 256   # 17 x 40 int32, rounded


def _cdiv(a, b):
    return -(-a // b)


def test_gemm_plan_invariants_random():
    """Random GEMM plans (1-12 projections, M 17-5000, N 1-20000, K up to the cap):
    the header's slot count, the order by K (longest first), contiguous slot ranges, and for every
    projection split along K (fewer than 128 tiles of 128 x 256, at least 32 stages
    of 128) ranges of an even number of stages, of at most about 16 unless the cap of one
    range-tile per compute unit binds, covering K exactly once; slices and zeros
    256-byte aligned, disjoint and filling the workspace exactly."""
    L = bt.lib()
    f = FAKE
    rng = np.random.default_rng(7)
    built = 0
    for trial in range(200):
        count = int(rng.integers(1, 13))
        shapes = [(int(rng.integers(17, 5001)), int(rng.integers(1, 20001)),
                   128 * int(rng.integers(1, 1025))) for _ in range(count)]
        m = (BtMatmulDesc * count)(*[BtMatmulDesc(mm, n, k, f, f, f, f, 0.02, f, None, None)
                                     for mm, n, k in shapes])
        need = L.bt_matmul_plan_workspace_bytes(m, count)
        nb = L.bt_matmul_plan_bytes(count)
        host = np.zeros(nb, np.uint8)
        base = 0x7E0000000000
        assert L.bt_matmul_plan_build(m, count, base, need, host.ctypes.data, nb) == OK, trial
        built += 1
        d = host[16:16 + 152 * count].reshape(count, 152)
        i32 = lambda i, o: int(d[i, o:o + 4].view(np.int32)[0])   # noqa: E731
        i64 = lambda i, o: int(d[i, o:o + 8].view(np.int64)[0])   # noqa: E731
        assert [i32(i, 60) for i in range(count)] == sorted((k for _, _, k in shapes), reverse=True), trial
        slot, pieces = 0, []
        for i in range(count):
            mm, n, k = i32(i, 52), i32(i, 56), i32(i, 60)
            splits, sps, slots, slot_begin = i32(i, 120), i32(i, 124), i32(i, 144), i32(i, 148)
            ws, ws_slice = i64(i, 128), i64(i, 136)
            tiles = _cdiv(mm, 128) * _cdiv(n, 256)
            nst = _cdiv(k, 128)
            assert slots == min(64, _cdiv(tiles, 8)) and slot_begin == slot, (trial, i)
            slot += slots * splits
            if tiles >= 128 or nst < 32:
                assert splits == 1 and ws == 0, (trial, i, splits)
                continue
            want = max(2, min(_cdiv(nst, 16), 256 // tiles))
            assert sps % 2 == 0 and sps == _cdiv(_cdiv(nst, want), 2) * 2, (trial, i, sps)
            assert (splits - 1) * sps < nst <= splits * sps, (trial, i)   # K covered once
            assert 2 <= splits <= want and splits * tiles <= 256, (trial, i)
            slice_bytes = _cdiv(mm * n * 4, 256) * 256
            assert ws_slice * 4 == slice_bytes and ws % 256 == 0, (trial, i)
            pieces.append((ws, splits * slice_bytes + _cdiv(mm * 4, 256) * 256))
        assert host[8:16].view(np.int64)[0] == slot, trial
        at = base
        for ws, size in sorted(pieces):
            assert ws == at, trial          # carved back to back from the start
            at += size
        assert at - base == need, trial
        if need:
            assert L.bt_matmul_plan_build(m, count, base, need - 1, host.ctypes.data, nb) \
                == WORKSPACE
    assert built == 200


def test_ternarize_plan_building_on_host():
    """A grouped ternarization plan: each tensor gets bt_ternarize's workspace
    slice and workgroup counts (first pass min(1024, ceil(N*K/4/2048)), second
    min(2048, ceil(N*K/16/256))) at consecutive offsets; bt_ternarize's argument
    errors, a missing workspace and overlapping outputs between tensors are
    reported before anything is written."""
    L = bt.lib()
    base = 0x7F0000000000
    shapes = [(2048, 1536), (17, 128), (1536, 8960)]
    addr = [base + (i << 32) for i in range(3)]      # far apart: no overlaps
    d = (BtTernarizeDesc * 3)(*[BtTernarizeDesc(a, n, k, 1e-5, a + (1 << 31), a + (1 << 31) + (1 << 30))
                                for a, (n, k) in zip(addr, shapes)])
    ws_each = [L.bt_ternarize_workspace_bytes(n, k) for n, k in shapes]
    need = L.bt_ternarize_plan_workspace_bytes(d, 3)
    assert need == sum(ws_each)
    nb = L.bt_ternarize_plan_bytes(3)
    assert nb == 16 + 3 * 80
    host = np.zeros(nb, np.uint8)
    wsb = base + (8 << 32)
    assert L.bt_ternarize_plan_build(d, 3, wsb, need - 1, host.ctypes.data, nb) == WORKSPACE
    assert not host.any()
    assert L.bt_ternarize_plan_build(d, 3, wsb, need, host.ctypes.data, nb) == OK
    assert host[:4].view(np.uint32)[0] == 0x42545454
    t = host[16:].reshape(3, 80)
    parts = [min(1024, -(-(n * k // 4) // 2048)) for n, k in shapes]
    packs = [min(2048, -(-(n * k // 16) // 256)) for n, k in shapes]
    assert host[8:16].view(np.int64)[0] == sum(parts)
    for i in range(3):
        assert t[i, 24:32].view(np.int64)[0] == wsb + sum(ws_each[:i])      # partials
        assert t[i, 52:56].view(np.int32)[0] == parts[i]
        assert t[i, 56:60].view(np.int32)[0] == packs[i]
        assert t[i, 64:72].view(np.int64)[0] == sum(parts[:i])
        assert t[i, 72:80].view(np.int64)[0] == sum(packs[:i])
    # errors, each leaving the plan unwritten
    for field, bad, want in (("K", 100, SHAPE), ("eps", -1.0, VALUE), ("eps", float("nan"), VALUE),
                             ("w", 0, NULL), ("packed", addr[1] + (1 << 31) + 4, ALIGN)):
        keep = getattr(d[1], field)
        setattr(d[1], field, bad)
        host[:] = 0
        assert L.bt_ternarize_plan_build(d, 3, wsb, need, host.ctypes.data, nb) == want, field
        assert not host.any(), field
        setattr(d[1], field, keep)
    # tensor 2's packed bytes inside tensor 0's weights
    keep = d[2].packed
    d[2].packed = addr[0] + 4096
    assert L.bt_ternarize_plan_build(d, 3, wsb, need, host.ctypes.data, nb) == VALUE
    d[2].packed = keep
    # the workspace inside a tensor's weights, or meeting another tensor's packed bytes
    assert L.bt_ternarize_plan_build(d, 3, addr[2], need, host.ctypes.data, nb) == VALUE
    assert L.bt_ternarize_plan_build(d, 3, addr[2] + (1 << 31) - 256, need, host.ctypes.data,
                                     nb) == VALUE
    # a launch with another plan kind is refused on the host
    host[:4] = np.frombuffer(np.uint32(0x42545141).tobytes(), np.uint8)
    assert L.bt_ternarize_grouped(host.ctypes.data, FAKE, None) == VALUE


def test_repack_plan_building_on_host():
    L = bt.lib()
    f = FAKE
    r = (BtRepackDesc * 3)(BtRepackDesc(f, f, 2048, 1536), BtRepackDesc(f, f, 40, 384),
                           BtRepackDesc(f, f, 1536, 8960))
    nb = L.bt_repack_plan_bytes(3)
    assert nb == 16 + 3 * 48
    host = np.zeros(nb, np.uint8)
    assert L.bt_repack_plan_build(r, 3, host.ctypes.data, nb) == OK
    assert host[:4].view(np.uint32)[0] == 0x4254504B
    # 1 KB output blocks: ceil(N/16) tiles x ceil(K/256) steps, summed
    blocks = 128 * 6 + 3 * 2 + 96 * 35
    assert host[8:16].view(np.int64)[0] == blocks
    # RepackDesc: 2 pointers, N, K, steps, pad (int32), then block_begin, blocks (int64)
    d = host[16:].reshape(3, 48)
    assert d[1, 32:40].view(np.int64)[0] == 128 * 6 and d[2, 40:48].view(np.int64)[0] == 96 * 35
    assert L.bt_repack_plan_build(r, 3, host.ctypes.data, nb - 1) == WORKSPACE
    assert L.bt_repack_plan_build(r, 0, host.ctypes.data, nb) == SHAPE
    r[1].K = 200                                 # K must be a multiple of 128
    assert L.bt_repack_plan_build(r, 3, host.ctypes.data, nb) == SHAPE
    r[1].K = 384
    r[2].wdev = f + 8
    assert L.bt_repack_plan_build(r, 3, host.ctypes.data, nb) == ALIGN
    r[2].wdev = None
    assert L.bt_repack_plan_build(r, 3, host.ctypes.data, nb) == NULL
    # a launch with a plan of the wrong kind is refused on the host
    q = (BtQuantDesc * 1)(BtQuantDesc(f, f, f, f, 3, 1536))
    qb = np.zeros(L.bt_quant_plan_bytes(1), np.uint8)
    assert L.bt_quant_plan_build(q, 1, qb.ctypes.data, qb.size) == OK
    assert L.bt_repack_ternary_grouped(qb.ctypes.data, f, None) == VALUE
    assert L.bt_repack_ternary_grouped(None, f, None) == NULL


def test_binding_has_no_cpu_fallback():
    import inspect
    import ternary_weight_decoder_bt_amd.ops as ops
    src = inspect.getsource(ops)
    assert "oracle" not in src and "import synth" not in src
    for host_math in ("np.dot", "np.matmul", "torch.matmul", "torch.mm", "np.round", "torch.round"):
        assert host_math not in src
