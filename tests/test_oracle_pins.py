"""Pins for the CPU oracle: checks against hand-derived values, closed forms,
special cases and brute force. None of these re-types the oracle's formulas.

Sources: "VibeVoice-ASR-BitNet Technical Report" sections 2.2.2 (ternary
weights in 2 bits, INT8 per-token activations, 8x less weight traffic than
FP16) and 2.4.2 / Figure 4 (integer vec_dot with exact hsum); the blog post
"Paper 說支援 ARM，我大概是第一個真的去編譯的人" (128-element groups whose
decode depends on the group size; a naive element-wise matmul as the exact
reference; a narrow accumulator that overflowed).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ternary_ref as tr
import synth


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- packing

def test_packed_size_is_one_eighth_of_fp16():
    for n, k in [(1, 128), (1536, 1536), (17920, 1536), (1536, 8960)]:
        w = np.zeros((n, k), np.int8) if n * k <= 4_000_000 else None
        assert oracle.packed_bytes(n, k) * 8 == n * k * 2
        if w is not None:
            assert oracle.pack_ref(w).nbytes * 8 == n * k * 2


def test_constant_rows_pack_to_hand_derived_bytes():
    k = 256
    for val, byte in [(1, 0xAA), (0, 0x55), (-1, 0x00)]:
        p = oracle.pack_ref(np.full((2, k), val, np.int8))
        assert p.shape == (2, k // 4)
        assert (p == byte).all()


def test_single_element_positions_match_golden(golden):
    rows = golden("pack_positions.txt")
    assert len(rows) >= 10
    for k_s, j_s, plus_s, minus_s in rows:
        k, j = int(k_s), int(j_s)
        for val, expect in [(1, int(plus_s, 16)), (-1, int(minus_s, 16))]:
            w = np.zeros((1, 256), np.int8)
            w[0, k] = val
            p = oracle.pack_ref(w)[0]
            assert p[j] == expect, (k, val)
            others = np.delete(p, j)
            assert (others == 0x55).all()


def test_roundtrip_random_and_every_position():
    rng = _rng(5)
    for n, k in [(3, 128), (7, 256), (16, 1536), (5, 8960)]:
        w = rng.integers(-1, 2, (n, k), dtype=np.int8)
        assert np.array_equal(oracle.unpack_ref(oracle.pack_ref(w), k), w)
    # every element position of one group, with each of the three values,
    # against a background of each other value
    for bg in (-1, 0, 1):
        for val in (-1, 0, 1):
            w = np.full((128, 128), bg, np.int8)
            w[np.arange(128), np.arange(128)] = val
            assert np.array_equal(oracle.unpack_ref(oracle.pack_ref(w), 128), w)


def test_no_code_three_ever_produced():
    w = _rng(6).integers(-1, 2, (64, 1024), dtype=np.int8)
    p = oracle.pack_ref(w)
    for s in range(4):
        assert ((p >> (2 * s)) & 3).max() <= 2


def test_pack_and_unpack_reject_bad_inputs():
    with pytest.raises(oracle.OracleError):
        oracle.pack_ref(np.zeros((2, 100), np.int8))
    with pytest.raises(oracle.OracleError):
        oracle.pack_ref(np.full((2, 128), 2, np.int8))
    p = np.full((1, 32), 0x55, np.uint8)
    p[0, 3] = 0x57                      # field 0 of byte 3 becomes 3
    with pytest.raises(oracle.OracleError):
        oracle.unpack_ref(p, 128)


def _decode_grouped_64(packed, k):
    """A wrong decoder: the same bit planes, but read with 64-element groups
    (16 bytes per group). The blog post's fourth bug was this reading."""
    n = packed.shape[0]
    g = packed.reshape(n, k // 64, 16)
    out = np.empty((n, k // 64, 4, 16), np.int8)
    for s in range(4):
        out[:, :, s, :] = ((g >> (2 * s)) & 3).astype(np.int8) - 1
    return out.reshape(n, k)


def test_negative_control_64_grouping_fails_parity():
    rng = _rng(7)
    w = rng.integers(-1, 2, (32, 256), dtype=np.int8)
    q = rng.integers(-127, 128, (4, 256), dtype=np.int8)
    wrong = _decode_grouped_64(oracle.pack_ref(w), 256)
    assert not np.array_equal(wrong, w)
    assert not np.array_equal(oracle.matmul_ref(q, wrong), oracle.matmul_ref(q, w))


def test_one_hot_rows_select_one_activation():
    rng = _rng(8)
    k, n = 384, 48
    q = rng.integers(-127, 128, (3, k), dtype=np.int8)
    kstar = rng.integers(0, k, n)
    sign = rng.choice([-1, 1], n)
    w = np.zeros((n, k), np.int8)
    w[np.arange(n), kstar] = sign
    w_rt = oracle.unpack_ref(oracle.pack_ref(w), k)
    acc = oracle.matmul_ref(q, w_rt)
    assert np.array_equal(acc, q[:, kstar].astype(np.int32) * sign[None, :])


@pytest.mark.parametrize("k", [128, 256])
def test_identity_weights_give_activations(k):
    q = _rng(9).integers(-127, 128, (5, k), dtype=np.int8)
    w_rt = oracle.unpack_ref(oracle.pack_ref(np.eye(k, dtype=np.int8)), k)
    assert np.array_equal(oracle.matmul_ref(q, w_rt), q.astype(np.int32))


# ------------------------------------------------------------- quantization

def test_quantize_matches_hand_worked_golden(golden):
    rows = golden("quantize_worked.txt")
    xs = {r[0]: np.array([np.float32(v) for v in r[2:]], np.float32) for r in rows if r[1] == "x"}
    qs = {r[0]: np.array([int(v) for v in r[2:]]) for r in rows if r[1] == "q"}
    labels = sorted(xs)
    x = np.stack([xs[l] for l in labels])
    q, d, qsum = oracle.quantize_ref(x)
    for i, l in enumerate(labels):
        assert np.array_equal(q[i].astype(int), qs[l]), l
        assert qsum[i] == qs[l].sum()
    assert d[labels.index("C")] == 0
    assert d[labels.index("B")] == np.float32(1.0)     # 127 / 127


def _exact_round_half_away(v: float) -> int:
    """Nearest integer to v with ties away from zero, in exact rational arithmetic."""
    f = Fraction(v)
    n = abs(f)
    fl = n.numerator // n.denominator
    r = fl + (1 if n - fl >= Fraction(1, 2) else 0)
    return r if f >= 0 else -r


def test_quantize_brute_force_rational():
    rng = _rng(10)
    x = rng.standard_normal((6, 200), dtype=np.float32)
    x[1] *= np.float32(1e-3)
    x[2, 17] = np.float32(40.0)          # an outlier row
    x[3] = rng.standard_t(3, 200).astype(np.float32)
    q, d, _ = oracle.quantize_ref(x)
    for m in range(x.shape[0]):
        a = max(abs(float(v)) for v in x[m])
        inv = np.float32(127) / np.float32(a)          # one IEEE fp32 division
        for kk in range(x.shape[1]):
            v = float(np.float32(x[m, kk]) * inv)      # one IEEE fp32 product
            expect = max(-127, min(127, _exact_round_half_away(v)))
            assert int(q[m, kk]) == expect
        # d * 127 reproduces a to within an ulp of a
        assert abs(float(d[m]) * 127 - a) <= float(np.spacing(np.float32(a)))


def test_quantize_extremes_map_to_127():
    rng = _rng(11)
    x = rng.standard_normal((8, 1536), dtype=np.float32)
    q, _, _ = oracle.quantize_ref(x)
    am = np.argmax(np.abs(x), axis=1)
    assert np.array_equal(q[np.arange(8), am], np.where(x[np.arange(8), am] > 0, 127, -127))
    assert np.abs(q.astype(int)).max() == 127
    assert q.min() >= -127


def test_quantize_sign_symmetry_and_scale_invariance():
    x = _rng(12).standard_normal((4, 512), dtype=np.float32)
    q1, d1, s1 = oracle.quantize_ref(x)
    q2, d2, s2 = oracle.quantize_ref(-x)
    assert np.array_equal(q2, -q1) and np.array_equal(d1, d2) and np.array_equal(s2, -s1)
    # scaling by a power of two is exact, so q cannot change
    q3, d3, _ = oracle.quantize_ref(x * np.float32(8))
    assert np.array_equal(q3, q1) and np.array_equal(d3, d1 * np.float32(8))


def test_quantize_tiny_absmax_rows():
    x = np.zeros((4, 128), np.float32)
    x[0, 5] = np.float32(1e-39)    # subnormal absmax: 127/a overflows
    x[1, 6] = np.float32(-1e-37)   # normal, but 127/a still overflows
    x[2, 7] = np.float32(1e-36)    # 127/a finite; d is subnormal
    x[2, 8] = np.float32(-5e-37)
    q, d, qs = oracle.quantize_ref(x)
    assert (q[0] == 0).all() and d[0] == 0
    assert (q[1] == 0).all() and d[1] == 0
    assert q[2, 7] == 127 and q[2, 8] in (-63, -64)
    assert 0 < d[2] < np.finfo(np.float32).tiny       # subnormal kept
    assert (q[3] == 0).all() and d[3] == 0 and qs[3] == 0


def test_quantize_rejects_non_finite():
    x = np.ones((1, 128), np.float32)
    x[0, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.quantize_ref(x)


# ---------------------------------------------------------------- matmul

def test_matmul_hand_worked_golden(golden):
    k = 128
    q = ((np.arange(k) % 5) - 2).astype(np.int8)[None, :]
    w = np.zeros((5, k), np.int8)
    w[0] = 1
    w[1, :64], w[1, 64:] = 1, -1
    w[2] = -1
    w[4, 7] = w[4, 8] = 1
    expect = {int(r): int(v) for r, v in golden("matmul_worked.txt")}
    for mode in ("loops", "int64", "f64"):
        acc = oracle.matmul_ref(q, w, mode)
        for r, v in expect.items():
            assert acc[0, r] == v, (mode, r)


def test_matmul_modes_agree_brute_force_tiny():
    rng = _rng(13)
    for m, n, k in [(1, 3, 128), (4, 8, 256), (3, 5, 128)]:
        q = rng.integers(-127, 128, (m, k), dtype=np.int8)
        w = rng.integers(-1, 2, (n, k), dtype=np.int8)
        a = oracle.matmul_ref(q, w, "loops")
        assert np.array_equal(a, oracle.matmul_ref(q, w, "int64"))
        assert np.array_equal(a, oracle.matmul_ref(q, w, "f64"))


def test_matmul_closed_forms():
    rng = _rng(14)
    k = 1536
    q = rng.integers(-127, 128, (3, k), dtype=np.int8)
    qs = q.astype(np.int64).sum(axis=1)
    w = np.stack([np.ones(k, np.int8), -np.ones(k, np.int8), np.zeros(k, np.int8)])
    acc = oracle.matmul_ref(q, w, "f64")
    assert np.array_equal(acc[:, 0], qs) and np.array_equal(acc[:, 1], -qs)
    assert (acc[:, 2] == 0).all()


def test_matmul_code_offset_identity():
    rng = _rng(15)
    q = rng.integers(-127, 128, (5, 256), dtype=np.int8)
    w = rng.integers(-1, 2, (9, 256), dtype=np.int8)
    codes = (w + 1).astype(np.int8)
    lhs = oracle.matmul_ref(q, codes).astype(np.int64) - q.astype(np.int64).sum(1)[:, None]
    assert np.array_equal(lhs, oracle.matmul_ref(q, w))


def test_matmul_worst_case_needs_int32():
    k = 8960
    q = np.full((1, k), 127, np.int8)
    w = np.ones((2, k), np.int8)
    w[1] = -1
    acc = oracle.matmul_ref(q, w, "f64")
    assert acc[0, 0] == 1_137_920 and acc[0, 1] == -1_137_920
    assert acc.dtype == np.int32
    assert 1_137_920 > np.iinfo(np.int16).max


def test_sampled_dot_products_match_full_matmul():
    rng = _rng(16)
    q = rng.integers(-127, 128, (6, 512), dtype=np.int8)
    w = rng.integers(-1, 2, (40, 512), dtype=np.int8)
    full = oracle.matmul_ref(q, w, "f64")
    rows, cols = rng.integers(0, 6, 50), rng.integers(0, 40, 50)
    assert np.array_equal(oracle.matmul_rows_cols(q, w, rows, cols), full[rows, cols])


# ---------------------------------------------------------------- rescale

def test_dequant_closed_form_values():
    acc = np.array([[1000, 0, -7]], np.int32)
    y = oracle.dequant_ref(acc, np.array([0.5], np.float32), 0.25)
    assert y.dtype == np.float32
    assert y[0, 0] == 125.0 and y[0, 1] == 0.0 and y[0, 2] == -0.875


def test_dequant_relative_error_bound():
    rng = _rng(17)
    acc = rng.integers(-1_137_920, 1_137_921, (8, 64)).astype(np.int32)
    d = rng.uniform(1e-3, 1.0, 8).astype(np.float32)
    s = np.float32(0.0312)
    y = oracle.dequant_ref(acc, d, s).astype(np.float64)
    exact = acc.astype(np.float64) * (d.astype(np.float64) * float(s))[:, None]
    nz = exact != 0
    assert (np.abs(y[nz] - exact[nz]) / np.abs(exact[nz])).max() <= 2 * 2.0 ** -24 * (1 + 1e-9)
    assert (y[~nz] == 0).all()


def test_forward_single_gemv_workload_end_to_end():
    c = synth.config0()
    out = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    assert out["acc"].shape == (1, 1536) and out["y"].dtype == np.float32
    # the float result approximates x @ W^T * s_w up to the INT8 quantization error
    ref = (c["x"].astype(np.float64) @ c["w"].astype(np.float64).T) * 0.02
    err = np.abs(out["y"] - ref)
    bound = float(out["d"][0]) * 0.5 * np.abs(c["w"]).sum(axis=1) * 0.02 * (1 + 1e-6)
    assert (err <= bound + 1e-6).all()


# -------------------------------------- the pins catch planted mistakes

def test_pins_detect_planted_half_to_even(monkeypatch, golden):
    monkeypatch.setattr(tr, "_round_half_away", lambda v: np.rint(v.astype(np.float64)))
    with pytest.raises(AssertionError):
        test_quantize_matches_hand_worked_golden(golden)


def test_pins_detect_planted_fp32_rounding(monkeypatch, golden):
    monkeypatch.setattr(tr, "_round_half_away",
                        lambda v: np.sign(v) * np.floor(np.abs(v) + np.float32(0.5)))
    with pytest.raises(AssertionError):
        test_quantize_matches_hand_worked_golden(golden)


def test_pins_detect_planted_sequential_layout(monkeypatch, golden):
    def seq_pack(w):
        codes = (w.astype(np.int16) + 1).astype(np.uint8)
        n, k = codes.shape
        c = codes.reshape(n, k // 4, 4)
        return (c[:, :, 0] | (c[:, :, 1] << 2) | (c[:, :, 2] << 4) | (c[:, :, 3] << 6)).astype(np.uint8)
    monkeypatch.setattr(oracle, "pack_ref", seq_pack)
    with pytest.raises(AssertionError):
        test_single_element_positions_match_golden(golden)
