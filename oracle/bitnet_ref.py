"""Plain CPU oracle for the offline ternarization of full-precision weights.

TEST INFRASTRUCTURE ONLY, like ``ternary_ref``: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it, and it imports
nothing from the HIP library or its binding.

What it follows:

* "VibeVoice-ASR-BitNet Technical Report", section 2.2.2: the decoder's weights
  are quantized to ternary {-1, 0, +1} following the BitNet approach of its
  reference [11] ("The era of 1-bit LLMs: all large language models are in
  1.58 bits"). The report does not print the quantizer itself.
* That cited paper's absmean quantizer, restated: the tensor's mean absolute
  value gamma is its scale; every weight is divided by gamma plus a small
  epsilon, rounded to the nearest integer and clipped to [-1, 1].

Readings where the pages are silent (each also listed in the design notes):

* Precision, step by step, so that every code is reproducible bit for bit:
  S = sum of |w| over the whole N x K tensor, the correctly rounded fp64 value
  of the exact sum (``math.fsum``); gamma = fl32(fl64(S / (N K)));
  delta = fl32(gamma + eps); t = fl32(w / delta) (IEEE division);
  code = clamp(round_half_away_from_zero(t), -1, 1). An implementation that
  sums in another order differs from S by far less than one fp32 unit of
  gamma; only a tensor whose S / (N K) lies that close to an fp32 rounding
  boundary can round gamma differently.
* Ties (t = +-0.5 exactly) round away from zero, as the activation quantizer
  of this library does.
* The per-tensor scale returned with the codes is gamma itself (W is
  approximated by gamma * code); eps only keeps the division finite.
* delta = 0 (an all-zero tensor with eps = 0) gives all codes 0 and gamma 0.
  (Otherwise |t| <= N K up to rounding, so the quotient never overflows.)

Pinned in tests/test_oracle_pins_ternarize.py by a hand-worked example
(tests/golden/ternarize_worked.txt), closed forms (constant magnitudes,
rows of different magnitudes under one per-tensor scale), power-of-two
scaling, and exact rational arithmetic on small random tensors.
"""

from __future__ import annotations

import math

import numpy as np

from .ternary_ref import GROUP_K, OracleError, pack_ref


def _round_half_away(v: np.ndarray) -> np.ndarray:
    """Nearest integer, ties away from zero (sign(v) * floor(|v| + 1/2), exact in fp64)."""
    v64 = np.asarray(v, dtype=np.float64)
    return np.sign(v64) * np.floor(np.abs(v64) + 0.5)


def absmean_ref(w: np.ndarray) -> np.float32:
    """gamma = fl32(fl64(S / (N K))), S the correctly rounded fp64 sum of |w|."""
    w64 = np.abs(np.asarray(w, dtype=np.float32).astype(np.float64)).reshape(-1)
    s = math.fsum(w64)
    return np.float32(s / w64.size)


def ternarize_ref(w: np.ndarray, eps: float):
    """fp32 W (N, K), eps >= 0 -> (int8 codes (N, K) in {-1, 0, 1}, fp32 gamma)."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[0] < 1 or w.shape[1] < 1:
        raise OracleError("weights must be a non-empty (N, K) matrix")
    if not np.isfinite(w).all():
        raise OracleError("weights must be finite")
    if not (math.isfinite(eps) and eps >= 0):
        raise OracleError("eps must be finite and >= 0")
    gamma = absmean_ref(w)
    delta = np.float32(gamma + np.float32(eps))
    if delta == 0:
        return np.zeros(w.shape, dtype=np.int8), np.float32(0)
    t = (w / delta).astype(np.float32)                     # fl32
    codes = np.clip(_round_half_away(t), -1, 1).astype(np.int8)
    return codes, gamma


def ternarize_pack_ref(w: np.ndarray, eps: float):
    """Ternarize, then pack in the canonical 2-bit format:
    (uint8 (N, K/4), fp32 gamma). K must be a multiple of 128."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % GROUP_K:
        raise OracleError(f"K must be a positive multiple of {GROUP_K}")
    codes, gamma = ternarize_ref(w, eps)
    return pack_ref(codes), gamma
