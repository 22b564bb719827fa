"""Pins for the offline-ternarization oracle (absmean quantizer of the BitNet
reference that "VibeVoice-ASR-BitNet Technical Report" section 2.2.2 follows):
a hand-worked example with ties, closed forms, per-tensor (not per-row)
scaling, exact power-of-two scaling and exact rational arithmetic. None
re-types the oracle's formulas.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import OracleError, pack_ref, unpack_ref
from oracle import bitnet_ref as tz


def _golden_matrix(golden):
    vals, c0, c25 = [], [], []
    for v, count, a, b in golden("ternarize_worked.txt"):
        vals += [float(v)] * int(count)
        c0 += [int(a)] * int(count)
        c25 += [int(b)] * int(count)
    assert len(vals) == 256
    shape = (2, 128)
    return (np.array(vals, np.float32).reshape(shape), np.array(c0, np.int8).reshape(shape),
            np.array(c25, np.int8).reshape(shape))


def test_hand_worked_golden_with_ties(golden):
    w, want0, want25 = _golden_matrix(golden)
    for eps, want in ((0.0, want0), (0.25, want25)):
        codes, gamma = tz.ternarize_ref(w, eps)
        assert gamma == np.float32(0.25)
        np.testing.assert_array_equal(codes, want)
    # the packed form unpacks to the same codes
    packed, gamma = tz.ternarize_pack_ref(w, 0.0)
    np.testing.assert_array_equal(unpack_ref(packed, 128), want0)
    np.testing.assert_array_equal(packed, pack_ref(want0))


def test_golden_layout_is_not_symmetric(golden):
    # the example must tell a transposed or reversed layout apart
    _, want0, _ = _golden_matrix(golden)
    assert not np.array_equal(want0[:, ::-1], want0)
    assert not np.array_equal(want0[::-1], want0)


@pytest.mark.parametrize("c", [1.0, 0.0078125, 3.5, 2.0 ** -60])
def test_constant_magnitude_gives_signs(c):
    # |w| = c everywhere: gamma = c exactly, every quotient is +-1
    rng = np.random.default_rng(3)
    s = rng.choice(np.array([-1, 1], np.int8), size=(7, 256))
    codes, gamma = tz.ternarize_ref(s.astype(np.float32) * np.float32(c), 0.0)
    assert gamma == np.float32(c)
    np.testing.assert_array_equal(codes, s)


def test_zeros_keep_their_code_and_shrink_gamma():
    # a fraction z of zeros and +-2 elsewhere: gamma = 2(1 - z) <= 2, every nonzero
    # quotient is >= 1 in magnitude, so codes = sign(w)
    w = np.zeros((4, 128), np.float32)
    w[:, ::4] = 2.0
    w[:, 1::4] = -2.0
    codes, gamma = tz.ternarize_ref(w, 0.0)
    assert gamma == np.float32(1.0)
    np.testing.assert_array_equal(codes, np.sign(w).astype(np.int8))


def test_scale_is_per_tensor_not_per_row():
    # row 0 at 1.0, row 1 at 0.25: gamma = 0.625 over the tensor, so row 1's
    # quotient is 0.4 -> 0 (a per-row scale would give 1 for both rows)
    w = np.stack([np.full(128, 1.0, np.float32), np.full(128, -0.25, np.float32)])
    codes, gamma = tz.ternarize_ref(w, 0.0)
    assert gamma == np.float32(0.625)
    assert (codes[0] == 1).all() and (codes[1] == 0).all()


@pytest.mark.parametrize("p", [-20, -3, 1, 7])
def test_power_of_two_scaling(p):
    # scaling by 2^p scales every step exactly: same codes, gamma * 2^p
    rng = np.random.default_rng(11)
    w = rng.standard_normal((5, 384)).astype(np.float32)
    c1, g1 = tz.ternarize_ref(w, 0.0)
    c2, g2 = tz.ternarize_ref(w * np.float32(2.0 ** p), 0.0)
    np.testing.assert_array_equal(c1, c2)
    assert g2 == np.float32(g1 * np.float32(2.0 ** p))


def test_exact_rational_decisions():
    # gamma from the exact rational mean; each code is the exact decision
    # wherever the exact quotient is not within 1e-6 of a rounding boundary
    rng = np.random.default_rng(5)
    for trial in range(6):
        n, k = rng.integers(1, 6), 128 * int(rng.integers(1, 3))
        w = (rng.standard_normal((n, k)) * rng.choice([0.01, 1.0, 30.0])).astype(np.float32)
        eps = [0.0, 1e-5, 0.01][trial % 3]
        codes, gamma = tz.ternarize_ref(w, eps)
        exact_mean = sum(Fraction(float(abs(v))) for v in w.reshape(-1)) / w.size
        assert abs(float(gamma) - float(exact_mean)) <= 2.0 ** -23 * float(exact_mean)
        denom = Fraction(float(np.float32(gamma + np.float32(eps))))
        checked = 0
        for idx, v in np.ndenumerate(w):
            t = Fraction(float(v)) / denom
            a = abs(t)
            if min(abs(a - Fraction(1, 2)), abs(a - Fraction(3, 2))) < Fraction(1, 10 ** 6):
                continue
            want = 0 if a < Fraction(1, 2) else (1 if t > 0 else -1)
            assert codes[idx] == want, (trial, idx, float(t))
            checked += 1
        assert checked > 0.99 * w.size


def test_all_zero_tensor():
    for eps in (0.0, 1e-5):
        codes, gamma = tz.ternarize_ref(np.zeros((3, 128), np.float32), eps)
        assert gamma == 0 and not codes.any()


def test_sum_beyond_fp32_range():
    # |w| sums to 6e38, past fp32's range: the fp64 sum keeps gamma finite, and
    # the two large weights' quotients (64) clip to +-1
    w = np.zeros((1, 128), np.float32)
    w[0, 0] = 3.0e38
    w[0, 1] = -3.0e38
    codes, gamma = tz.ternarize_ref(w, 0.0)
    assert codes[0, 0] == 1 and codes[0, 1] == -1 and not codes[0, 2:].any()
    assert gamma == np.float32(6.0e38 / 128)


@pytest.mark.parametrize("bad", [
    dict(w=np.zeros((2, 128), np.float32), eps=-1.0),
    dict(w=np.zeros((2, 128), np.float32), eps=float("nan")),
    dict(w=np.full((2, 128), np.inf, np.float32), eps=0.0),
    dict(w=np.zeros((0, 128), np.float32), eps=0.0),
])
def test_domain_errors(bad):
    with pytest.raises(OracleError):
        tz.ternarize_ref(bad["w"], bad["eps"])


def test_pack_needs_whole_groups():
    with pytest.raises(OracleError):
        tz.ternarize_pack_ref(np.ones((2, 100), np.float32), 0.0)
