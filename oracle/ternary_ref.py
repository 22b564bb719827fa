"""Plain CPU oracle for the ternary-weight x INT8-activation matmul.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it, and this module imports nothing from the
product path: the two share no code. It is written for clarity, not speed:
NumPy element-wise arithmetic in the precision each step is defined in.

What it follows (pages cited by title and section):

* "VibeVoice-ASR-BitNet Technical Report", section 2.2.2 (I2_S): the decoder's
  linear-layer weights take values in {-1, 0, +1} and are stored in 2 bits;
  activations are quantized to INT8 online, per token; the kernel unpacks the
  ternary codes to INT8 and runs an integer multiply-add.
* Same report, section 2.4.2 and Figure 4: N x 1 parallel vec_dot, each output
  is one weight row dotted with the activation vector; products are summed in
  integers (maddubs -> madd -> hsum).
* Blog post "Paper 說支援 ARM，我大概是第一個真的去編譯的人", second postscript:
  the weight file stores ternary codes in 128-element groups, and decoding them
  with a 64-element grouping scrambles the matrix. So the bit layout inside a
  group depends on the group size: it is interleaved.
* Same post, fourth stage: a naive element-wise matmul is the semantic
  reference; an optimized kernel must match it bit for bit.

Readings where the pages are silent (each also listed in the design notes):

* Activation scheme: per-token absmax, symmetric, no zero point; range
  [-127, 127]; round half away from zero.
* Code of a weight: w + 1 (so -1 -> 0, 0 -> 1, +1 -> 2); the 2-bit field 3 is
  invalid. Four codes per byte. Byte b of 128-element group g holds elements
  128g + b, 128g + 32 + b, 128g + 64 + b, 128g + 96 + b in bits 0-1, 2-3, 4-5,
  6-7 (least significant pair first).
* Scales: one fp32 scale per weight tensor; d_m = a_m / 127 per token; the fp32
  output is fl32(fl32(acc) * fl32(d_m * s_w)).
* An all-zero row, or a row whose 127/a overflows, quantizes to zeros with
  d = 0 (so its output is exactly 0).

Every function here is pinned by tests that do not re-type its formulas:
hand-derived byte values, closed forms, textbook special cases and brute force
(tests/test_oracle_pins.py).
"""

from __future__ import annotations

import numpy as np

GROUP_K = 128          # elements per packed group along K
SUB = 32               # bytes per group = elements per bit-pair plane
QMAX = 127


class OracleError(ValueError):
    """An input outside the method's domain (bad shape, value or code)."""


# --------------------------------------------------------------------------
# Packing (technical report section 2.2.2; blog post, second postscript)
# --------------------------------------------------------------------------

def packed_bytes(n: int, k: int) -> int:
    """Bytes of the 2-bit format: N*K/4, i.e. one eighth of the FP16 matrix."""
    return n * k // 4


def pack_ref(w: np.ndarray) -> np.ndarray:
    """int8 W (N, K) with values in {-1, 0, +1} -> uint8 (N, K/4) canonical bytes.

    For row n, group g, bit-pair plane s in 0..3 and byte b in 0..31:
    packed[n, 32g + b] holds code(w[n, 128g + 32s + b]) = w + 1 at bits 2s..2s+1.
    """
    w = np.asarray(w)
    if w.ndim != 2:
        raise OracleError("weights must be 2-D (N, K)")
    n, k = w.shape
    if n < 1 or k < 1 or k % GROUP_K:
        raise OracleError(f"K={k} must be a positive multiple of {GROUP_K}")
    if not np.isin(w, (-1, 0, 1)).all():
        raise OracleError("weights must be in {-1, 0, +1}")
    codes = (w.astype(np.int16) + 1).astype(np.uint8)          # 0, 1, 2
    planes = codes.reshape(n, k // GROUP_K, 4, SUB)             # [n, g, s, b]
    packed = np.zeros((n, k // GROUP_K, SUB), dtype=np.uint8)   # [n, g, b]
    for s in range(4):
        packed |= (planes[:, :, s, :] << np.uint8(2 * s)).astype(np.uint8)
    return packed.reshape(n, k // 4)


def unpack_ref(packed: np.ndarray, k: int) -> np.ndarray:
    """Exact inverse of :func:`pack_ref`. A 2-bit field equal to 3 is an error."""
    packed = np.asarray(packed, dtype=np.uint8)
    if k % GROUP_K or packed.ndim != 2 or packed.shape[1] != k // 4:
        raise OracleError("packed buffer does not match K")
    n = packed.shape[0]
    grouped = packed.reshape(n, k // GROUP_K, SUB)
    planes = np.empty((n, k // GROUP_K, 4, SUB), dtype=np.uint8)
    for s in range(4):
        planes[:, :, s, :] = (grouped >> np.uint8(2 * s)) & np.uint8(3)
    if (planes == 3).any():
        raise OracleError("2-bit code 3 does not encode a ternary value")
    return (planes.reshape(n, k).astype(np.int16) - 1).astype(np.int8)


# --------------------------------------------------------------------------
# Per-token INT8 activation quantization (technical report section 2.2.2)
# --------------------------------------------------------------------------

def _round_half_away(v32: np.ndarray) -> np.ndarray:
    """sign(v) * floor(|v| + 1/2), evaluated exactly.

    v is fp32; widening to fp64 makes |v| + 1/2 exact for every |v| that can
    round to a non-zero integer, so no second rounding can push a value just
    below one half up to one.
    """
    v = v32.astype(np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def quantize_ref(x: np.ndarray):
    """fp32 x (M, K) -> (q int8 (M, K), d fp32 (M,), qsum int32 (M,)).

    Per row m, each arithmetic step in IEEE fp32 with round-to-nearest-even:
      a = max_k |x[m, k]|;  inv = fl32(127 / a);
      if a == 0 or inv is not finite: q = 0, d = 0;
      else q = clamp(round_half_away(fl32(x * inv)), -127, 127), d = fl32(a / 127).
    qsum[m] = sum_k q[m, k].
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[0] < 1 or x.shape[1] < 1:
        raise OracleError("activations must be a non-empty (M, K) matrix")
    if not np.isfinite(x).all():
        raise OracleError("activations must be finite")
    a = np.max(np.abs(x), axis=1)                                   # exact
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.float32(QMAX) / a                                   # fl32
    dead = (a == 0) | ~np.isfinite(inv)
    inv = np.where(dead, np.float32(0), inv).astype(np.float32)
    v = (x * inv[:, None]).astype(np.float32)                        # fl32
    q = np.clip(_round_half_away(v), -QMAX, QMAX)
    q[dead] = 0
    d = (a / np.float32(QMAX)).astype(np.float32)                    # fl32
    d[dead] = 0
    q = q.astype(np.int8)
    return q, d, q.astype(np.int64).sum(axis=1).astype(np.int32)


# --------------------------------------------------------------------------
# Integer matmul (technical report section 2.4.2, Figure 4)
# --------------------------------------------------------------------------

def matmul_loops(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * w[n, k], one Python-int product at a time.

    The naive element-wise reference; for tiny shapes only.
    """
    m_, k = q.shape
    n_, k2 = w.shape
    assert k == k2
    acc = np.zeros((m_, n_), dtype=np.int64)
    for m in range(m_):
        for n in range(n_):
            s = 0
            for kk in range(k):
                s += int(q[m, kk]) * int(w[n, kk])
            acc[m, n] = s
    return acc


def matmul_int64(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Exact integer matmul in int64 (NumPy's integer product, no BLAS)."""
    return q.astype(np.int64) @ w.astype(np.int64).T


def matmul_f64(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Exact integer matmul through an fp64 GEMM.

    Exact because every partial sum is an integer of magnitude at most
    127 * K <= 127 * 8960 < 2**24 < 2**53.
    """
    k = q.shape[1]
    assert QMAX * k < 2 ** 53
    acc = q.astype(np.float64) @ w.astype(np.float64).T
    out = np.rint(acc).astype(np.int64)
    assert np.array_equal(out.astype(np.float64), acc)
    return out


def matmul_ref(q: np.ndarray, w: np.ndarray, mode: str = "int64") -> np.ndarray:
    """int32 acc (M, N); checks |acc| <= 127 * K."""
    fn = {"loops": matmul_loops, "int64": matmul_int64, "f64": matmul_f64}[mode]
    acc = fn(q, w)
    assert np.abs(acc).max(initial=0) <= QMAX * q.shape[1]
    return acc.astype(np.int32)


def matmul_rows_cols(q: np.ndarray, w: np.ndarray, rows, cols) -> np.ndarray:
    """acc at sampled (row, col) pairs: one int64 dot product per pair."""
    return np.array([int(q[r].astype(np.int64) @ w[c].astype(np.int64))
                     for r, c in zip(rows, cols)], dtype=np.int64).astype(np.int32)


# --------------------------------------------------------------------------
# Rescale to fp32
# --------------------------------------------------------------------------

def dequant_ref(acc: np.ndarray, d: np.ndarray, w_scale) -> np.ndarray:
    """y[m, n] = fl32(fl32(acc[m, n]) * fl32(d_m * s_w)); fl32(acc) is exact (|acc| < 2**24)."""
    acc = np.asarray(acc)
    assert np.abs(acc).max(initial=0) < 2 ** 24
    rs = (np.asarray(d, dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    return (acc.astype(np.float32) * rs[:, None]).astype(np.float32)


def forward_ref(x: np.ndarray, w: np.ndarray, w_scale, mode: str = "int64") -> dict:
    """The whole path on one projection: quantize, integer matmul, rescale."""
    q, d, qsum = quantize_ref(x)
    acc = matmul_ref(q, w, mode)
    return {"q": q, "d": d, "qsum": qsum, "acc": acc, "y": dequant_ref(acc, d, w_scale)}
