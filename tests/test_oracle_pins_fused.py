"""Pins for the fused-operator oracle (RMS normalization with scale, then the
per-token INT8 quantization): hand-worked values, closed forms, exact scaling
laws and an error bound against the exact real result. None re-types the
oracle's formulas.

Sources: "VibeVoice-ASR-BitNet Technical Report" section 2.4.1
(rms_norm_scaled, a fused RMS normalization with a scale parameter) and
section 2.2.2 (INT8 activations per token).
"""

from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import fused_ref as fused


def _cases(golden):
    cases = {}
    for r in golden("rmsnorm_worked.txt"):
        kind, case = r[0], r[1]
        c = cases.setdefault(case, {"rows": {}})
        if kind == "g":
            c["g"] = np.array(r[2:], np.float32)
        elif kind == "eps":
            c["eps"] = float(r[2])
        else:
            c["rows"].setdefault(r[2], {})[kind] = np.array(r[3:], np.float64)
    return cases


def test_rmsnorm_matches_hand_worked_golden(golden):
    for case in _cases(golden).values():
        labels = sorted(case["rows"])
        x = np.array([case["rows"][l]["x"] for l in labels], np.float32)
        h = fused.rmsnorm_scaled_ref(x, case["g"], case["eps"])
        q, d, s = fused.rmsnorm_quantize_ref(x, case["g"], case["eps"])
        for i, l in enumerate(labels):
            row = case["rows"][l]
            assert np.array_equal(h[i], row["h"].astype(np.float32)), (l, h[i])
            assert np.array_equal(q[i], row["q"].astype(np.int8)), (l, q[i])
            assert s[i] == int(row["qsum"][0])
            a = np.float32(np.max(np.abs(row["h"])))
            assert d[i] == (a / np.float32(127) if a else 0)


def test_rmsnorm_constant_rows_closed_form():
    # power-of-two constants with eps = 0: every step is exact, h = sign(c) * g
    g = np.random.default_rng(3).standard_normal(96).astype(np.float32)
    for c in (1.0, -0.25, 2.0 ** 20, -(2.0 ** -20), 64.0):
        x = np.full((1, 96), c, np.float32)
        assert np.array_equal(fused.rmsnorm_scaled_ref(x, g, 0.0)[0], np.sign(c) * g)


def test_rmsnorm_eps_sits_inside_the_root():
    # mean square 1 plus eps 3 = 4, root 2: h = g / 2 exactly; with eps 12, root 3.6...
    g = np.linspace(-2, 2, 8).astype(np.float32)
    x = np.ones((1, 8), np.float32)
    assert np.array_equal(fused.rmsnorm_scaled_ref(x, g, 3.0)[0], g / 2)
    # mean square 4 (x = 2) plus eps 12 = 16, root 4: h = x/4 * g = g / 2
    assert np.array_equal(fused.rmsnorm_scaled_ref(2 * x, g, 12.0)[0], g / 2)


def test_rmsnorm_power_of_two_scaling_is_exact():
    # with eps = 0, scaling a row by 2^p scales S by 4^p, the root by 2^p and
    # r by 2^-p, all exactly, so h does not change at all
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 200)).astype(np.float32)
    g = rng.uniform(0.5, 2, 200).astype(np.float32)
    h = fused.rmsnorm_scaled_ref(x, g, 0.0)
    for p in (-6, 3, 10):
        assert np.array_equal(fused.rmsnorm_scaled_ref(x * np.float32(2.0 ** p), g, 0.0), h)


def test_rmsnorm_rows_are_independent_and_zero_rows_give_zero():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    g = rng.uniform(0.5, 2, 64).astype(np.float32)
    x[2] = 0
    h = fused.rmsnorm_scaled_ref(x, g, 1e-6)
    for i in range(5):
        assert np.array_equal(fused.rmsnorm_scaled_ref(x[i:i + 1], g, 1e-6)[0], h[i])
    assert (h[2] == 0).all()
    q, d, s = fused.rmsnorm_quantize_ref(x, g, 0.0)     # eps 0: the zero row's r is not finite
    assert (q[2] == 0).all() and d[2] == 0 and s[2] == 0


def test_rmsnorm_within_a_few_ulp_of_the_exact_result():
    # the exact real h = x / sqrt(sum(x^2)/K + eps) * g, evaluated with 40-digit
    # decimals; the oracle rounds five times (mean, sum with eps, root,
    # reciprocal, two products), so it must lie within 8 fp32 ulp of it
    getcontext().prec = 40
    rng = np.random.default_rng(6)
    for k, eps in ((7, 0.0), (33, 1e-6), (128, 0.5)):
        x = (rng.standard_normal((3, k)) * 3).astype(np.float32)
        g = rng.uniform(-2, 2, k).astype(np.float32)
        h = fused.rmsnorm_scaled_ref(x, g, eps)
        for i in range(3):
            ss = sum(Decimal(float(v)) ** 2 for v in x[i])
            root = (ss / k + Decimal(float(np.float32(eps)))).sqrt()
            for j in range(k):
                exact = Decimal(float(x[i, j])) / root * Decimal(float(g[j]))
                ulp = np.spacing(np.float32(abs(float(exact)) or 1e-30))
                assert abs(Decimal(float(h[i, j])) - exact) <= 8 * Decimal(float(ulp))


def test_rmsnorm_rejects_bad_inputs():
    x = np.ones((2, 8), np.float32)
    g = np.ones(8, np.float32)
    for bad in (lambda: fused.rmsnorm_scaled_ref(x, g[:4], 0.0),
                lambda: fused.rmsnorm_scaled_ref(x, g, -1.0),
                lambda: fused.rmsnorm_scaled_ref(x, g, float("nan")),
                lambda: fused.rmsnorm_scaled_ref(np.full((2, 8), np.inf, np.float32), g, 0.0)):
        with pytest.raises(fused.OracleError):
            bad()


# -------------------------------------- the pins catch planted mistakes

def _planted(monkeypatch, scale):
    monkeypatch.setattr(fused, "rmsnorm_scale", scale)


def test_pins_detect_planted_eps_outside_the_root(monkeypatch, golden):
    def wrong(x, eps):
        ms = (fused.rmsnorm_sumsq(x) / x.shape[1]).astype(np.float32)
        with np.errstate(divide="ignore"):
            r = (np.float32(1) / (np.sqrt(ms).astype(np.float32) + np.float32(eps))).astype(np.float32)
        return np.where(np.isfinite(r), r, 0).astype(np.float32)
    _planted(monkeypatch, wrong)
    with pytest.raises(AssertionError):
        test_rmsnorm_matches_hand_worked_golden(golden)


def test_pins_detect_planted_sum_instead_of_mean(monkeypatch):
    def wrong(x, eps):
        s = fused.rmsnorm_sumsq(x).astype(np.float32)
        with np.errstate(divide="ignore"):
            r = (np.float32(1) / np.sqrt(s + np.float32(eps)).astype(np.float32)).astype(np.float32)
        return np.where(np.isfinite(r), r, 0).astype(np.float32)
    _planted(monkeypatch, wrong)
    with pytest.raises(AssertionError):
        test_rmsnorm_constant_rows_closed_form()


# ------------------------------------------------------------- epilogues

def _epi_golden(golden):
    return {r[0]: np.array(r[1:], np.float64) for r in golden("epilogue_worked.txt")}


def test_epilogue_matches_hand_worked_golden(golden):
    from oracle import ternary_ref as tr
    v = _epi_golden(golden)
    y = tr.dequant_ref(v["acc"].astype(np.int64)[None, :], np.float32(v["d"]), np.float32(v["s_w"]))
    assert np.array_equal(y[0], v["y"].astype(np.float32))
    b, gm, res = (v[k].astype(np.float32) for k in ("bias", "gamma", "residual"))
    assert np.array_equal(fused.epilogue_ref(y, bias=b, relu=True)[0], v["bias_relu"])
    assert np.array_equal(fused.epilogue_ref(y, b, True, gm, res[None, :])[0], v["all"])
    assert np.array_equal(fused.epilogue_ref(y, b, False, gm, res[None, :])[0], v["all_no_relu"])


def test_epilogue_closed_forms():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((4, 50)).astype(np.float32)
    assert np.array_equal(fused.epilogue_ref(y), y)                                  # identity
    assert (fused.epilogue_ref(-np.abs(y) - 1, relu=True) == 0).all()                # ReLU
    assert np.array_equal(fused.epilogue_ref(np.abs(y), relu=True), np.abs(y))
    assert np.array_equal(fused.epilogue_ref(y, layer_scale=np.full(50, 0.25, np.float32)),
                          y / 4)                                                     # exact 2^-2
    assert np.array_equal(fused.epilogue_ref(y, residual=np.zeros_like(y)), y)
    # integers stay exact through every step
    yi = rng.integers(-1000, 1000, (3, 20)).astype(np.float32)
    bi = rng.integers(-50, 50, 20).astype(np.float32)
    gi = rng.integers(-4, 5, 20).astype(np.float32)
    ri = rng.integers(-9, 9, (3, 20)).astype(np.float32)
    want = ri + gi * np.maximum(yi + bi, 0)
    assert np.array_equal(fused.epilogue_ref(yi, bi, True, gi, ri), want)


def test_pins_detect_planted_scale_after_residual(monkeypatch, golden):
    def wrong(y, bias=None, relu=False, layer_scale=None, residual=None):
        out = y + bias if bias is not None else y
        out = np.maximum(out, 0) if relu else out
        out = out + residual if residual is not None else out
        return (out * layer_scale).astype(np.float32) if layer_scale is not None else out
    monkeypatch.setattr(fused, "epilogue_ref", wrong)
    with pytest.raises(AssertionError):
        test_epilogue_matches_hand_worked_golden(golden)


def test_epilogue_relu_gives_positive_zero():
    y = np.array([[-0.0, 0.0, -1e-30, 2.0]], np.float32)
    out = fused.epilogue_ref(y, relu=True)
    assert np.array_equal(out, [[0, 0, 0, 2]]) and not np.signbit(out).any()
