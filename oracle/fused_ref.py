"""Plain CPU oracle for the operators fused around the ternary matmul.

TEST INFRASTRUCTURE ONLY, like ``ternary_ref``: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it, and it imports
nothing from the HIP library or its binding.

What it follows (pages cited by title and section):

* "VibeVoice-ASR-BitNet Technical Report", section 2.4.1 (operator fusion): a
  fused RMS normalization with a scale parameter (``rms_norm_scaled``) is one
  of the fused operators, and section 2.4.2 ("Other kernels") pairs INT8 RMS
  normalization with the GEMM kernels. Section 2.2.2: the decoder's linear
  layers quantize their activations to INT8 per token, which makes the
  normalization that precedes a projection and that quantization one pass.

Readings where the pages are silent (each also listed in the design notes):

* RMS normalization is the textbook one: h = x / sqrt(mean_k(x^2) + eps) * g,
  with g one fp32 scale per channel (the "scale parameter") and eps >= 0.
* Precision, step by step, so that the quantization decision downstream is
  reproducible bit for bit: the sum of squares is taken in fp64 (each fp32
  square is exact in fp64) and rounded once: ms = fl32(S / K);
  r = fl32(1 / fl32(sqrt(fl32(ms + eps)))); a row whose r is not finite (an
  all-zero row with eps = 0, or squares that vanish in fp32) gets r = 0, so
  h = 0; h = fl32(fl32(x * r) * g). The quantization of h is ``quantize_ref``.
* S is the correctly rounded fp64 value of the exact sum (``math.fsum``); an
  implementation that sums in another order differs from it by far less than
  one fp32 unit of ms, and only a row whose S lies that close to an fp32
  rounding boundary can round ms differently.

* The fused epilogues of section 2.4.1 applied to the matmul's fp32 output y:
  ``mul_mat_add_relu`` (matrix multiply + bias + ReLU) and ``add_scaled``
  (residual addition with layer-scale multiplication). Order and precision,
  each step one fp32 operation: y1 = fl32(y + bias[n]); y2 = y1 if y1 > 0
  else +0;
  y3 = fl32(gamma[n] * y2); out = fl32(residual[m, n] + y3). The layer scale
  multiplies the branch before the residual is added, as in the ConvNeXt
  blocks the report's tokenizer is built from (section 2.2.1). Every step is
  optional.

Every function here is pinned in tests/test_oracle_pins_fused.py by closed
forms (constant rows, power-of-two scalings, eps inside the root, exact small
integers through the epilogue) and hand-worked examples
(tests/golden/rmsnorm_worked.txt, tests/golden/epilogue_worked.txt), not by
re-typed formulas.
"""

from __future__ import annotations

import math

import numpy as np

from .ternary_ref import OracleError, quantize_ref


def rmsnorm_sumsq(x: np.ndarray) -> np.ndarray:
    """S[m] = sum_k x[m, k]^2, correctly rounded to fp64 (exact squares, fsum)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    return np.array([math.fsum(row * row) for row in x64], dtype=np.float64)


def rmsnorm_scale(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-row fp32 factor r = fl32(1 / fl32(sqrt(fl32(ms + eps)))), ms = fl32(S / K).

    Rows whose r is not finite get r = 0.
    """
    x = np.asarray(x, dtype=np.float32)
    k = x.shape[1]
    ms = (rmsnorm_sumsq(x) / k).astype(np.float32)
    t = (ms + np.float32(eps)).astype(np.float32)
    root = np.sqrt(t).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        r = (np.float32(1) / root).astype(np.float32)
    return np.where(np.isfinite(r), r, np.float32(0)).astype(np.float32)


def rmsnorm_scaled_ref(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """fp32 x (M, K), fp32 g (K,), eps >= 0 -> fp32 h (M, K) = fl32(fl32(x * r) * g)."""
    x = np.asarray(x, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    if x.ndim != 2 or x.shape[0] < 1 or x.shape[1] < 1:
        raise OracleError("activations must be a non-empty (M, K) matrix")
    if g.shape != (x.shape[1],):
        raise OracleError("the scale must hold one value per channel")
    if not (np.isfinite(x).all() and np.isfinite(g).all()):
        raise OracleError("activations and scale must be finite")
    if not (math.isfinite(eps) and eps >= 0):
        raise OracleError("eps must be finite and >= 0")
    r = rmsnorm_scale(x, eps)
    return ((x * r[:, None]).astype(np.float32) * g[None, :]).astype(np.float32)


def rmsnorm_quantize_ref(x: np.ndarray, g: np.ndarray, eps: float):
    """RMS normalization with scale, then the per-token INT8 quantization:
    (q int8 (M, K), d fp32 (M,), qsum int32 (M,))."""
    return quantize_ref(rmsnorm_scaled_ref(x, g, eps))


def epilogue_ref(y: np.ndarray, bias=None, relu: bool = False, layer_scale=None,
                 residual=None) -> np.ndarray:
    """fp32 y (M, N) -> fp32 out (M, N): bias add, ReLU, layer scale, residual add,
    in that order, each optional and each one fp32 operation."""
    y = np.asarray(y, dtype=np.float32)
    if y.ndim != 2:
        raise OracleError("y must be (M, N)")
    n = y.shape[1]
    out = y
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float32)
        if bias.shape != (n,):
            raise OracleError("bias must hold one value per output")
        out = (out + bias[None, :]).astype(np.float32)
    if relu:
        # y if y > 0 else +0: a negative zero comes out as +0
        out = np.where(out > 0, out, np.float32(0)).astype(np.float32)
    if layer_scale is not None:
        layer_scale = np.asarray(layer_scale, dtype=np.float32)
        if layer_scale.shape != (n,):
            raise OracleError("the layer scale must hold one value per output")
        out = (layer_scale[None, :] * out).astype(np.float32)
    if residual is not None:
        residual = np.asarray(residual, dtype=np.float32)
        if residual.shape != y.shape:
            raise OracleError("the residual must have the output's shape")
        out = (residual + out).astype(np.float32)
    return out
