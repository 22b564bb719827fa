"""Pins for the I8_S oracle (int8 x int8): brute force, closed forms, extreme
magnitudes, and agreement with the ternary oracle on ternary weights. None
re-types the oracle's formula.

Sources: "VibeVoice-ASR-BitNet Technical Report" section 2.2.1 (I8_S, an INT8
datapath) and section 2.4.2 / Figure 4 (one integer multiply-add pipeline for
I8_S and I2_S).
"""

import numpy as np
import pytest

import oracle
from oracle import i8s_ref


def test_i8s_brute_force_tiny():
    rng = np.random.default_rng(1)
    for m, n, k in ((1, 1, 1), (2, 3, 5), (4, 7, 32)):
        q = rng.integers(-127, 128, (m, k), dtype=np.int8)
        w = rng.integers(-128, 128, (n, k), dtype=np.int8)
        want = [[sum(int(q[i, j]) * int(w[c, j]) for j in range(k)) for c in range(n)]
                for i in range(m)]
        assert np.array_equal(i8s_ref.i8s_matmul_ref(q, w), np.array(want))


def test_i8s_closed_forms():
    rng = np.random.default_rng(2)
    q = rng.integers(-127, 128, (3, 64), dtype=np.int8)
    eye = np.eye(64, dtype=np.int8)
    assert np.array_equal(i8s_ref.i8s_matmul_ref(q, eye), q)          # identity
    onehot = np.zeros((2, 64), np.int8)
    onehot[0, 5], onehot[1, 63] = -128, 127
    acc = i8s_ref.i8s_matmul_ref(q, onehot)
    assert np.array_equal(acc[:, 0], -128 * q[:, 5].astype(np.int32))
    assert np.array_equal(acc[:, 1], 127 * q[:, 63].astype(np.int32))


def test_i8s_extreme_magnitude_needs_int32():
    k = 4096
    q = np.full((1, k), -127, np.int8)
    w = np.full((2, k), -128, np.int8)
    w[1] = 127
    acc = i8s_ref.i8s_matmul_ref(q, w)
    assert acc[0, 0] == 127 * 128 * k and acc[0, 1] == -127 * 127 * k
    assert abs(int(acc[0, 0])) > 2 ** 15 * 1000          # far beyond an int16 stage


def test_i8s_agrees_with_ternary_on_ternary_weights():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 256)).astype(np.float32)
    w = rng.integers(-1, 2, (9, 256), dtype=np.int8)
    t = oracle.forward_ref(x, w, np.float32(0.03), "int64")
    i = i8s_ref.i8s_forward_ref(x, w, np.float32(0.03))
    for key in ("q", "d", "acc", "y"):
        assert np.array_equal(t[key], i[key])


def test_i8s_rejects_bad_inputs():
    q = np.zeros((2, 8), np.int8)
    with pytest.raises(oracle.OracleError):
        i8s_ref.i8s_matmul_ref(q, np.zeros((3, 8), np.int16))
    with pytest.raises(oracle.OracleError):
        i8s_ref.i8s_matmul_ref(q, np.zeros((3, 7), np.int8))
