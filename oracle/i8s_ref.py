"""Plain CPU oracle for the I8_S product (int8 weights x int8 activations).

TEST INFRASTRUCTURE ONLY, like ``ternary_ref``: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it, and it imports
nothing from the HIP library or its binding.

What it follows (pages cited by title and section):

* "VibeVoice-ASR-BitNet Technical Report", section 2.2.1 (I8_S): weights,
  activations and every operator boundary of the tokenizer are INT8; section
  2.4.2 and Figure 4: the I8_S and I2_S kernels share one integer
  multiply-add pipeline (maddubs -> madd -> hsum), I2_S only adding the 2-bit
  unpack in front. So the product is the ternary one with int8 weights.

Readings where the pages are silent (each also listed in the design notes):

* Weights are int8 over the whole range [-128, 127] with one fp32 scale per
  tensor; activations are the per-token absmax INT8 codes of ``quantize_ref``.
* The product is exact: acc[m, n] = sum_k q[m, k] * w[n, k] in integers, and
  |acc| <= 127 * 128 * K, so K <= 131072 keeps it inside int32.
* The output at the kernel boundary is the same fp32 rescale as I2_S,
  fl32(fl32(acc) * fl32(d_m * s_w)); the next operator quantizes it again.

Pinned in tests/test_oracle_pins_i8s.py by brute force on tiny shapes, closed
forms (identity, one-hot rows, the extreme magnitudes) and the relation to the
ternary product on weights that happen to be ternary.
"""

from __future__ import annotations

import numpy as np

from .ternary_ref import OracleError, dequant_ref, quantize_ref

I8_KMAX = 131072   # 127 * 128 * K < 2**31


def i8s_matmul_ref(q: np.ndarray, w8: np.ndarray) -> np.ndarray:
    """int8 q (M, K) x int8 w8 (N, K) -> exact int32 acc (M, N), via int64."""
    q = np.asarray(q)
    w8 = np.asarray(w8)
    if q.dtype != np.int8 or w8.dtype != np.int8:
        raise OracleError("both operands must be int8")
    if q.ndim != 2 or w8.ndim != 2 or q.shape[1] != w8.shape[1]:
        raise OracleError("shapes must be (M, K) and (N, K)")
    if q.shape[1] > I8_KMAX:
        raise OracleError("K too large for an exact int32 sum")
    acc = q.astype(np.int64) @ w8.astype(np.int64).T
    assert np.abs(acc).max(initial=0) <= 127 * 128 * q.shape[1]
    return acc.astype(np.int32)


def i8s_forward_ref(x: np.ndarray, w8: np.ndarray, w_scale) -> dict:
    """The whole I8_S projection: quantize x per token, exact product, fp32 rescale."""
    q, d, qsum = quantize_ref(x)
    acc = i8s_matmul_ref(q, w8)
    return {"q": q, "d": d, "qsum": qsum, "acc": acc, "y": dequant_ref(acc, d, w_scale)}
