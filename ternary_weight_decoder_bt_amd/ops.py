"""Python binding of the bt C ABI: argument marshalling only.

Every computation runs in libbt (host packing in C++, everything else in HIP
kernels). PyTorch supplies device memory and the current HIP stream; NumPy
arrays carry host buffers.
"""

from __future__ import annotations

import ctypes as C

import numpy as np

from ._lib import (BtEpilogue, BtMatmulDesc, BtQuantDesc, BtRepackDesc, BtTernarizeDesc, BtError,
                   check, lib)

GROUP_K = 128
GEMV_MAX_M = 16


def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dev(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# ------------------------------------------------------------------ sizes

def packed_bytes(n: int, k: int) -> int:
    return int(lib().bt_packed_bytes(n, k))


def repacked_bytes(n: int, k: int) -> int:
    return int(lib().bt_repacked_bytes(n, k))


def matmul_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().bt_matmul_workspace_bytes(m, n, k))


# ------------------------------------------------------------- host format

def pack_ternary(w: np.ndarray) -> np.ndarray:
    """int8 (N, K) in {-1,0,1} -> canonical uint8 (N, K/4) (host, bt_pack_ternary)."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    if w.ndim != 2:
        raise ValueError("w must be (N, K)")
    n, k = w.shape
    out = np.empty((n, max(k // 4, 0)), np.uint8)
    check(lib().bt_pack_ternary(_np_ptr(w), n, k, _np_ptr(out)), "bt_pack_ternary")
    return out


def unpack_ternary(packed: np.ndarray, k: int) -> np.ndarray:
    """Canonical uint8 (N, K/4) -> int8 (N, K) (host, bt_unpack_ternary)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    if packed.shape[1] != k // 4:
        raise ValueError("packed width must be K/4")
    out = np.empty((n, k), np.int8)
    check(lib().bt_unpack_ternary(_np_ptr(packed), n, k, _np_ptr(out)), "bt_unpack_ternary")
    return out


# ------------------------------------------------------------------ device

def ternarize_workspace_bytes(n: int, k: int) -> int:
    return int(lib().bt_ternarize_workspace_bytes(n, k))


def ternarize(w, eps: float = 0.0, packed=None, scale=None, workspace=None, stream=None):
    """fp32 device W (N, K) -> (uint8 canonical packed bytes (N*K/4,), fp32 scale (1,))
    via bt_ternarize (absmean ternarization, codes packed as bt_pack_ternary does)."""
    torch = _torch()
    _dev(w, torch.float32, None, "w")
    if w.dim() != 2:
        raise ValueError("w must be (N, K)")
    n, k = w.shape
    nbytes = packed_bytes(n, k)
    if nbytes == 0:
        raise ValueError(f"invalid weight shape N={n}, K={k} (K must be a multiple of 128)")
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=w.device)
    _dev(packed, torch.uint8, (nbytes,), "packed")
    _dev(scale, torch.float32, (1,), "scale")
    need = ternarize_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=w.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib().bt_ternarize(_ptr(w), n, k, float(eps), _ptr(packed), _ptr(scale),
                             _ptr(workspace), ws_bytes, _stream(stream)), "bt_ternarize")
    return packed, scale


def repack_ternary(packed_dev, n: int, k: int, out=None, stream=None):
    """Canonical bytes on the device -> the kernels' tile layout (bt_repack_ternary)."""
    torch = _torch()
    _dev(packed_dev, torch.uint8, None, "packed_dev")
    if packed_dev.numel() != packed_bytes(n, k):
        raise ValueError("packed_dev must hold N*K/4 bytes")
    nbytes = repacked_bytes(n, k)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=packed_dev.device)
    _dev(out, torch.uint8, (nbytes,), "out")
    check(lib().bt_repack_ternary(_ptr(packed_dev), n, k, _ptr(out), _stream(stream)),
          "bt_repack_ternary")
    return out


def quantize_act(x, xq=None, xscale=None, xsum=None, stream=None):
    """fp32 (M, K) -> (int8 (M, K), fp32 (M,), int32 (M,)) via bt_quantize_act."""
    torch = _torch()
    _dev(x, torch.float32, None, "x")
    if x.dim() != 2:
        raise ValueError("x must be (M, K)")
    m, k = x.shape
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if xscale is None:
        xscale = torch.empty(m, dtype=torch.float32, device=x.device)
    if xsum is None:
        xsum = torch.empty(m, dtype=torch.int32, device=x.device)
    _dev(xq, torch.int8, (m, k), "xq")
    _dev(xscale, torch.float32, (m,), "xscale")
    _dev(xsum, torch.int32, (m,), "xsum")
    check(lib().bt_quantize_act(_ptr(x), m, k, _ptr(xq), _ptr(xscale), _ptr(xsum),
                                _stream(stream)), "bt_quantize_act")
    return xq, xscale, xsum


def rmsnorm_quantize(x, g, eps: float, xq=None, xscale=None, xsum=None, stream=None):
    """RMS normalization with per-channel scale g, then per-token INT8 quantization,
    in one launch (bt_rmsnorm_quantize): returns (int8 (M, K), fp32 (M,), int32 (M,))."""
    torch = _torch()
    _dev(x, torch.float32, None, "x")
    if x.dim() != 2:
        raise ValueError("x must be (M, K)")
    m, k = x.shape
    _dev(g, torch.float32, (k,), "g")
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if xscale is None:
        xscale = torch.empty(m, dtype=torch.float32, device=x.device)
    if xsum is None:
        xsum = torch.empty(m, dtype=torch.int32, device=x.device)
    _dev(xq, torch.int8, (m, k), "xq")
    _dev(xscale, torch.float32, (m,), "xscale")
    _dev(xsum, torch.int32, (m,), "xsum")
    check(lib().bt_rmsnorm_quantize(_ptr(x), _ptr(g), float(eps), m, k, _ptr(xq), _ptr(xscale),
                                    _ptr(xsum), _stream(stream)), "bt_rmsnorm_quantize")
    return xq, xscale, xsum


def new_workspace(m: int, n: int, k: int, device="cuda"):
    """Zero-filled workspace for bt_ternary_matmul (None when none is needed)."""
    torch = _torch()
    nbytes = matmul_workspace_bytes(m, n, k)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def ternary_matmul(xq, xscale, xsum, wdev, n: int, w_scale: float, y=None, acc=None,
                   workspace=None, want_acc=False, stream=None, bias=None, relu=False,
                   layer_scale=None, residual=None):
    """y = (xq @ W^T) * xscale * w_scale via bt_ternary_matmul; returns y (and acc).

    bias, relu, layer_scale, residual: the fused epilogue (bt_ternary_matmul_epilogue),
    y = residual + layer_scale * relu(y + bias); residual may be y itself.
    """
    torch = _torch()
    _dev(xq, torch.int8, None, "xq")
    m, k = xq.shape
    _dev(xscale, torch.float32, (m,), "xscale")
    _dev(xsum, torch.int32, (m,), "xsum")
    _dev(wdev, torch.uint8, (repacked_bytes(n, k),), "wdev")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _dev(y, torch.float32, (m, n), "y")
    if acc is None and want_acc:
        acc = torch.empty((m, n), dtype=torch.int32, device=xq.device)
    if acc is not None:
        _dev(acc, torch.int32, (m, n), "acc")
    need = matmul_workspace_bytes(m, n, k)
    if need and workspace is None:
        workspace = new_workspace(m, n, k, xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if bias is None and not relu and layer_scale is None and residual is None:
        check(lib().bt_ternary_matmul(m, n, k, _ptr(xq), _ptr(xscale), _ptr(xsum), _ptr(wdev),
                                      float(w_scale), _ptr(y), _ptr(acc), _ptr(workspace),
                                      ws_bytes, _stream(stream)), "bt_ternary_matmul")
    else:
        for t, shp, name in ((bias, (n,), "bias"), (layer_scale, (n,), "layer_scale"),
                             (residual, (m, n), "residual")):
            if t is not None:
                _dev(t, torch.float32, shp, name)
        epi = BtEpilogue(_ptr(bias), _ptr(layer_scale), _ptr(residual), 1 if relu else 0, 0)
        check(lib().bt_ternary_matmul_epilogue(m, n, k, _ptr(xq), _ptr(xscale), _ptr(xsum),
                                               _ptr(wdev), float(w_scale), C.byref(epi), _ptr(y),
                                               _ptr(acc), _ptr(workspace), ws_bytes,
                                               _stream(stream)), "bt_ternary_matmul_epilogue")
    return (y, acc) if (want_acc or acc is not None) else y


def ternary_matmul_noalloc(xq, xscale, xsum, wdev, n: int, w_scale: float, y, acc=None,
                           stream=None):
    """bt_ternary_matmul_noalloc: the same product with the split-K partial sums in
    the library's own device array (no workspace argument, nothing allocated by the
    call). y (and acc, if given) must be preallocated by the caller."""
    torch = _torch()
    _dev(xq, torch.int8, None, "xq")
    m, k = xq.shape
    _dev(xscale, torch.float32, (m,), "xscale")
    _dev(xsum, torch.int32, (m,), "xsum")
    _dev(wdev, torch.uint8, (repacked_bytes(n, k),), "wdev")
    _dev(y, torch.float32, (m, n), "y")
    if acc is not None:
        _dev(acc, torch.int32, (m, n), "acc")
    check(lib().bt_ternary_matmul_noalloc(m, n, k, _ptr(xq), _ptr(xscale), _ptr(xsum),
                                          _ptr(wdev), float(w_scale), _ptr(y), _ptr(acc),
                                          _stream(stream)), "bt_ternary_matmul_noalloc")
    return (y, acc) if acc is not None else y


def ternary_matmul_fused(x, wdev, n: int, w_scale: float, y=None, acc=None, xq=None,
                         xscale=None, xsum=None, workspace=None, want_acc=False, stream=None):
    """Quantize x and multiply in one launch (bt_ternary_matmul_fused, M <= 16).

    xq, xscale, xsum are optional outputs (same values as quantize_act).
    """
    torch = _torch()
    _dev(x, torch.float32, None, "x")
    m, k = x.shape
    _dev(wdev, torch.uint8, (repacked_bytes(n, k),), "wdev")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, (m, n), "y")
    if acc is None and want_acc:
        acc = torch.empty((m, n), dtype=torch.int32, device=x.device)
    for t, dt, shp, name in ((acc, torch.int32, (m, n), "acc"), (xq, torch.int8, (m, k), "xq"),
                             (xscale, torch.float32, (m,), "xscale"),
                             (xsum, torch.int32, (m,), "xsum")):
        if t is not None:
            _dev(t, dt, shp, name)
    need = matmul_workspace_bytes(m, n, k)
    if need and workspace is None:
        workspace = new_workspace(m, n, k, x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().bt_ternary_matmul_fused(m, n, k, _ptr(x), _ptr(wdev), float(w_scale), _ptr(y),
                                        _ptr(acc), _ptr(xq), _ptr(xscale), _ptr(xsum),
                                        _ptr(workspace), ws_bytes, _stream(stream)),
          "bt_ternary_matmul_fused")
    return (y, acc) if (want_acc or acc is not None) else y


# -------------------------------------------------------------------- I8_S

def int8_repacked_bytes(n: int, k: int) -> int:
    return int(lib().bt_int8_repacked_bytes(n, k))


def repack_int8(w_dev, out=None, stream=None):
    """int8 (N, K) weights on the device -> the kernels' tile layout (bt_repack_int8)."""
    torch = _torch()
    _dev(w_dev, torch.int8, None, "w_dev")
    if w_dev.dim() != 2:
        raise ValueError("w_dev must be (N, K)")
    n, k = w_dev.shape
    nbytes = int8_repacked_bytes(n, k)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w_dev.device)
    _dev(out, torch.uint8, (nbytes,), "out")
    check(lib().bt_repack_int8(_ptr(w_dev), n, k, _ptr(out), _stream(stream)), "bt_repack_int8")
    return out


def int8_matmul_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().bt_int8_matmul_workspace_bytes(m, n, k))


def int8_matmul(xq, xscale, w8dev, n: int, w_scale: float, y=None, acc=None, want_acc=False,
                stream=None, bias=None, relu=False, layer_scale=None, residual=None,
                workspace=None):
    """The I8_S product y = (xq @ W8^T) * xscale * w_scale (bt_int8_matmul), with the
    optional fused epilogue; returns y (and acc)."""
    torch = _torch()
    _dev(xq, torch.int8, None, "xq")
    m, k = xq.shape
    _dev(xscale, torch.float32, (m,), "xscale")
    _dev(w8dev, torch.uint8, (int8_repacked_bytes(n, k),), "w8dev")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _dev(y, torch.float32, (m, n), "y")
    if acc is None and want_acc:
        acc = torch.empty((m, n), dtype=torch.int32, device=xq.device)
    if acc is not None:
        _dev(acc, torch.int32, (m, n), "acc")
    epi = None
    if bias is not None or relu or layer_scale is not None or residual is not None:
        for t, shp, name in ((bias, (n,), "bias"), (layer_scale, (n,), "layer_scale"),
                             (residual, (m, n), "residual")):
            if t is not None:
                _dev(t, torch.float32, shp, name)
        epi = BtEpilogue(_ptr(bias), _ptr(layer_scale), _ptr(residual), 1 if relu else 0, 0)
    need = int8_matmul_workspace_bytes(m, n, k)
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=xq.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().bt_int8_matmul(m, n, k, _ptr(xq), _ptr(xscale), _ptr(w8dev), float(w_scale),
                               None if epi is None else C.byref(epi), _ptr(y), _ptr(acc),
                               _ptr(workspace), ws_bytes, _stream(stream)), "bt_int8_matmul")
    return (y, acc) if (want_acc or acc is not None) else y


# ------------------------------------------------------------------ grouped

class _Plan:
    def __init__(self, host: np.ndarray, device):
        torch = _torch()
        self.host = host
        self.dev = torch.from_numpy(host).to(device)
        torch.cuda.current_stream(device).synchronize()

    def _ptrs(self):
        return _np_ptr(self.host), _ptr(self.dev)


class RepackPlan(_Plan):
    """Many device repacks in one launch (bt_repack_ternary_grouped).

    items: sequence of (packed_dev, n, k, out) with out a uint8 CUDA tensor of
    repacked_bytes(n, k) bytes.
    """

    def __init__(self, items):
        torch = _torch()
        descs = (BtRepackDesc * len(items))()
        self._keep = list(items)
        for i, (packed, n, k, out) in enumerate(items):
            _dev(packed, torch.uint8, None, "packed_dev")
            if packed.numel() != packed_bytes(n, k):
                raise ValueError("packed_dev must hold N*K/4 bytes")
            _dev(out, torch.uint8, (repacked_bytes(n, k),), "out")
            descs[i] = BtRepackDesc(_ptr(packed), _ptr(out), n, k)
        nbytes = int(lib().bt_repack_plan_bytes(len(items)))
        host = np.zeros(nbytes, np.uint8)
        check(lib().bt_repack_plan_build(descs, len(items), _np_ptr(host), nbytes),
              "bt_repack_plan_build")
        super().__init__(host, items[0][0].device)

    def launch(self, stream=None):
        h, d = self._ptrs()
        check(lib().bt_repack_ternary_grouped(h, d, _stream(stream)), "bt_repack_ternary_grouped")


class TernarizePlan(_Plan):
    """Many offline ternarizations in one pair of launches (bt_ternarize_grouped).

    items: sequence of (w, packed, scale) CUDA tensors (fp32 (N, K), uint8
    (N*K/4,), fp32 (1,)); eps as for ternarize. The plan owns its workspace.
    """

    def __init__(self, items, eps: float = 0.0):
        torch = _torch()
        descs = (BtTernarizeDesc * len(items))()
        self._keep = list(items)
        for i, (w, packed, scale) in enumerate(items):
            _dev(w, torch.float32, None, "w")
            if w.dim() != 2:
                raise ValueError("w must be (N, K)")
            n, k = w.shape
            _dev(packed, torch.uint8, (packed_bytes(n, k),), "packed")
            _dev(scale, torch.float32, (1,), "scale")
            descs[i] = BtTernarizeDesc(_ptr(w), n, k, float(eps), _ptr(packed), _ptr(scale))
        dev = items[0][0].device
        ws_bytes = int(lib().bt_ternarize_plan_workspace_bytes(descs, len(items)))
        self.workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        nbytes = int(lib().bt_ternarize_plan_bytes(len(items)))
        host = np.zeros(nbytes, np.uint8)
        check(lib().bt_ternarize_plan_build(descs, len(items), _ptr(self.workspace), ws_bytes,
                                            _np_ptr(host), nbytes), "bt_ternarize_plan_build")
        super().__init__(host, dev)

    def launch(self, stream=None):
        h, d = self._ptrs()
        check(lib().bt_ternarize_grouped(h, d, _stream(stream)), "bt_ternarize_grouped")


class QuantPlan(_Plan):
    """Many independent quantizations in one launch (bt_quantize_act_grouped).

    items: sequence of (x, xq, xscale, xsum) CUDA tensors.
    """

    def __init__(self, items):
        descs = (BtQuantDesc * len(items))()
        self._keep = list(items)
        for i, (x, xq, xs, xsum) in enumerate(items):
            m, k = x.shape
            descs[i] = BtQuantDesc(_ptr(x), _ptr(xq), _ptr(xs), _ptr(xsum), m, k)
        nbytes = int(lib().bt_quant_plan_bytes(len(items)))
        host = np.zeros(nbytes, np.uint8)
        check(lib().bt_quant_plan_build(descs, len(items), _np_ptr(host), nbytes),
              "bt_quant_plan_build")
        super().__init__(host, items[0][0].device)

    def launch(self, stream=None):
        h, d = self._ptrs()
        check(lib().bt_quantize_act_grouped(h, d, _stream(stream)), "bt_quantize_act_grouped")


class MatmulPlan(_Plan):
    """Many independent projections in one launch (bt_ternary_matmul_grouped):
    all GEMVs (M <= 16) or all GEMMs (M > 16).

    items: sequence of dicts with keys wdev, n, w_scale, y, optionally acc, and
    either xq, xscale, xsum (quantized inputs) or, GEMVs only, x (fp32
    activations quantized inside the launch; xq, xscale, xsum then optional
    outputs). The plan owns the workspace its split projections need.
    """

    def __init__(self, items):
        descs = (BtMatmulDesc * len(items))()
        self._keep = list(items)
        for i, it in enumerate(items):
            src = it.get("x")
            m, k = (src if src is not None else it["xq"]).shape
            descs[i] = BtMatmulDesc(m, it["n"], k, _ptr(it.get("xq")), _ptr(it.get("xscale")),
                                    _ptr(it.get("xsum")), _ptr(it["wdev"]), float(it["w_scale"]),
                                    _ptr(it["y"]), _ptr(it.get("acc")), _ptr(src))
        torch = _torch()
        dev = items[0]["y"].device
        ws_bytes = int(lib().bt_matmul_plan_workspace_bytes(descs, len(items)))
        self.workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        nbytes = int(lib().bt_matmul_plan_bytes(len(items)))
        host = np.zeros(nbytes, np.uint8)
        check(lib().bt_matmul_plan_build(descs, len(items), _ptr(self.workspace), ws_bytes,
                                         _np_ptr(host), nbytes), "bt_matmul_plan_build")
        super().__init__(host, dev)

    def launch(self, stream=None):
        h, d = self._ptrs()
        check(lib().bt_ternary_matmul_grouped(h, d, _stream(stream)), "bt_ternary_matmul_grouped")


__all__ = [
    "BtError", "GROUP_K", "GEMV_MAX_M", "packed_bytes", "repacked_bytes",
    "matmul_workspace_bytes", "int8_repacked_bytes", "repack_int8", "int8_matmul", "int8_matmul_workspace_bytes", "pack_ternary", "unpack_ternary", "repack_ternary",
    "quantize_act", "rmsnorm_quantize", "new_workspace", "ternary_matmul", "ternary_matmul_noalloc",
    "ternary_matmul_fused", "RepackPlan", "TernarizePlan",
    "QuantPlan", "MatmulPlan",
]
