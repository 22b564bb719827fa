"""GPU parity for the operators fused around the ternary matmul, through the C
ABI, against the CPU oracle (oracle/fused_ref.py).

RMS normalization + quantization: q, d and the row sums bit-exact. The one
place an exact match is not implied by the definition is the fp64 sum of
squares, whose summation order is free: a row whose sum lies so close to an
fp32 rounding boundary of ms that the order could decide it is reported and
skipped (none is expected in these tests; at most one in a hundred rows may
be so flagged).
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import ternary_weight_decoder_bt_amd as bt  # noqa: E402

POISON_I32 = np.iinfo(np.int32).min


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def ambiguous_rows(x):
    """Rows whose ms = fl32(S/K) could round differently under another fp64
    summation order (relative change of S up to 1e-12)."""
    k = x.shape[1]
    s = oracle.rmsnorm_sumsq(x)
    lo = (s * (1 - 1e-12) / k).astype(np.float32)
    hi = (s * (1 + 1e-12) / k).astype(np.float32)
    return lo != hi


def run(x, g, eps, dev):
    m, k = x.shape
    xq = torch.full((m, k), 99, dtype=torch.int8, device=dev)
    xs = torch.full((m,), float("nan"), dtype=torch.float32, device=dev)
    xsum = torch.full((m,), POISON_I32, dtype=torch.int32, device=dev)
    bt.rmsnorm_quantize(to_dev(x, dev), to_dev(g, dev), eps, xq, xs, xsum)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy(), xsum.cpu().numpy()


def check(x, g, eps, dev):
    q, d, s = run(x, g, eps, dev)
    rq, rd, rs = oracle.rmsnorm_quantize_ref(x, g, eps)
    skip = ambiguous_rows(x)
    assert skip.mean() <= 0.01
    ok = ~skip
    assert np.array_equal(q[ok], rq[ok]), np.argwhere(q[ok] != rq[ok])[:3]
    assert np.array_equal(d[ok], rd[ok])
    assert np.array_equal(s[ok], rs[ok])
    # the skipped rows are still well-formed: row sums agree with the codes
    assert np.array_equal(s, q.astype(np.int64).sum(axis=1))


# wave-per-row path (K % 4 == 0, K <= 2048), block path in registers (K <= 9216),
# and the three-pass path (K % 4 != 0, or K > 9216)
@pytest.mark.parametrize("m,k", [(1, 1536), (7, 1536), (33, 2048), (5, 4100), (16, 8960),
                                 (3, 9216), (2, 9220), (4, 130), (3, 1)])
@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_rmsnorm_quantize_shapes(dev, m, k, eps):
    c = synth.small_problem(20, m, 16, max(k, 128), "outlier")
    rng = np.random.default_rng(m * 10000 + k)
    x = np.ascontiguousarray(c["x"][:, :k])
    g = rng.uniform(0.5, 1.5, k).astype(np.float32)
    check(x, g, eps, dev)


def test_rmsnorm_quantize_zero_tiny_and_constant_rows(dev):
    k = 1536
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, k)).astype(np.float32)
    x[1] = 0                      # zero row: r not finite at eps = 0 -> q = 0, d = 0
    x[2] = 1e-30                  # squares vanish in fp32 but not in fp64
    x[3] = -0.25                  # constant power of two: h = -g exactly
    x[4, :] = 0
    x[4, 7] = 3.0                 # one non-zero element
    g = rng.uniform(-2, 2, k).astype(np.float32)
    for eps in (0.0, 1e-6, 3.0):
        check(x, g, eps, dev)
        check(x[:, :130].copy(), g[:130].copy(), eps, dev)


@pytest.mark.parametrize("k", [1536, 8960])
def test_rmsnorm_quantize_long_prefill_rows(dev, k):
    """Full-size prefill activations (M = 4096, Student-t(3)), every row compared."""
    proj = 0 if k == 1536 else 3
    x = synth.long_prefill_problem(0, proj, with_weights=False)["x"]
    g = np.random.default_rng(k).uniform(0.5, 1.5, k).astype(np.float32)
    check(x, g, 1e-6, dev)


def test_rmsnorm_quantize_feeds_the_matmul(dev):
    """The fused output drives the ternary matmul to the oracle's result."""
    c = synth.small_problem(22, 9, 200, 1536, "normal")
    g = np.random.default_rng(22).uniform(0.5, 1.5, 1536).astype(np.float32)
    q, d, s = run(c["x"], g, 1e-6, dev)
    h = oracle.rmsnorm_scaled_ref(c["x"], g, 1e-6)
    ref = oracle.forward_ref(h, c["w"], c["w_scale"], "f64")
    assert np.array_equal(q, ref["q"]) and np.array_equal(d, ref["d"])
    packed = to_dev(bt.pack_ternary(c["w"]).reshape(-1), dev)
    wdev = bt.repack_ternary(packed, 200, 1536)
    y, acc = bt.ternary_matmul(to_dev(q, dev), to_dev(d, dev), to_dev(s, dev), wdev, 200,
                               c["w_scale"], want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert np.array_equal(y.cpu().numpy(), ref["y"])


# ------------------------------------------------------------- epilogues

def load_weights(w, dev):
    n, k = w.shape
    return bt.repack_ternary(to_dev(bt.pack_ternary(w).reshape(-1), dev), n, k)


EPILOGUES = {
    "bias_relu": dict(bias=True, relu=True),
    "scale_residual": dict(layer_scale=True, residual=True),
    "all": dict(bias=True, relu=True, layer_scale=True, residual=True),
    "relu_only": dict(relu=True),
}


# (4000, 1530, 256): 128 x 96 tiles (direct stores), ragged M and N
@pytest.mark.parametrize("m,n,k", [(1, 200, 384), (5, 1536, 1536), (16, 130, 8960),
                                   (40, 200, 384), (300, 1536, 1536), (4133, 4100, 384),
                                   (4096, 1540, 256), (4000, 1530, 256)])
@pytest.mark.parametrize("kind", list(EPILOGUES))
def test_matmul_epilogues(dev, m, n, k, kind):
    """GEMV (M <= 16), GEMM full and ragged tiles, with each epilogue; y against
    the oracle bit for bit, acc still the plain sum."""
    spec = EPILOGUES[kind]
    c = synth.small_problem(30, m, n, k, "t3", (0.3, 0.4, 0.3))
    rng = np.random.default_rng(m + n + k)
    bias = rng.standard_normal(n).astype(np.float32) if spec.get("bias") else None
    gamma = rng.uniform(-2, 2, n).astype(np.float32) if spec.get("layer_scale") else None
    res = rng.standard_normal((m, n)).astype(np.float32) if spec.get("residual") else None
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    want = oracle.epilogue_ref(ref["y"], bias, spec.get("relu", False), gamma, res)
    xq, xs, xsum = (to_dev(ref[k_], dev) for k_ in ("q", "d", "qsum"))
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
    bt.ternary_matmul(xq, xs, xsum, load_weights(c["w"], dev), n, c["w_scale"], y=y, acc=acc,
                      bias=None if bias is None else to_dev(bias, dev),
                      relu=spec.get("relu", False),
                      layer_scale=None if gamma is None else to_dev(gamma, dev),
                      residual=None if res is None else to_dev(res, dev))
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    bad = ~((got == want) | (np.isnan(got) & np.isnan(want)))
    assert not bad.any(), (np.argwhere(bad)[:3], got[bad][:3], want[bad][:3])
    if spec.get("relu") and not spec.get("layer_scale"):
        assert not np.signbit(got).any()          # ReLU gives +0, never -0


@pytest.mark.parametrize("m,n,k", [(3, 200, 384), (4096, 2048, 256), (4000, 1536, 256)])
def test_matmul_residual_in_place(dev, m, n, k):
    """residual = y: out = y_old + layer_scale * relu(y + bias), written over y_old."""
    c = synth.small_problem(31, m, n, k, "normal")
    rng = np.random.default_rng(31)
    old = rng.standard_normal((m, n)).astype(np.float32)
    bias = rng.standard_normal(n).astype(np.float32)
    gamma = rng.uniform(-2, 2, n).astype(np.float32)
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    want = oracle.epilogue_ref(ref["y"], bias, True, gamma, old)
    xq, xs, xsum = (to_dev(ref[k_], dev) for k_ in ("q", "d", "qsum"))
    y = to_dev(old, dev)
    bt.ternary_matmul(xq, xs, xsum, load_weights(c["w"], dev), n, c["w_scale"], y=y,
                      bias=to_dev(bias, dev), relu=True, layer_scale=to_dev(gamma, dev),
                      residual=y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), want)
