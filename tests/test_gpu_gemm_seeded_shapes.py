"""Dispatch over seeded random shapes: whatever the library picks (GEMV with or
without a K split; GEMM tile shape 128 x 256 persistent or tiled, 128 x 128,
128 x 96, 64 x 64, with or without a K split; for int8 weights also the
LDS-resident small-matrix kernel), the int32 sums match the oracle exactly and
y bit for bit, every output compared (NaN / poison-filled outputs, so an
unwritten element fails). Shapes have ragged M, N and K and are sized so the
oracle finishes each in about a second or less."""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import ternary_weight_decoder_bt_amd as bt  # noqa: E402

POISON_I32 = np.iinfo(np.int32).min


def seeded_shapes(seed=2026):
    """Three regimes, so that every tile shape and the split are exercised:
    wide outputs over a short K (persistent / 128 x 256 tiles), mid-sized
    outputs (128 x 128, 128 x 96, 64 x 64 tiles) and small outputs over a long K
    (64 x 64 tiles, K split)."""
    rng = np.random.default_rng(seed)
    regimes = (  # count, M range, N range, K/128 range, max M*N*K
        (8, (3000, 6000), (3500, 6000), (1, 4), 3.2e10),
        (10, (700, 3000), (600, 3000), (1, 24), 6e9),
        (10, (17, 700), (1, 3000), (8, 71), 3e9),
    )
    out = []
    for count, (m0, m1), (n0, n1), (k0, k1), cap in regimes:
        got = 0
        while got < count:
            m, n = int(rng.integers(m0, m1)), int(rng.integers(n0, n1))
            k = 128 * int(rng.integers(k0, k1 + 1))
            if m * n * k <= cap:
                out.append((m, n, k))
                got += 1
    return out


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("m,n,k", seeded_shapes())
def test_gemm_seeded_shape(dev, m, n, k):
    c = synth.small_problem(77, m, n, k, "t3", (0.25, 0.5, 0.25))
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    xq, xs, xsum = (to_dev(ref[k_], dev) for k_ in ("q", "d", "qsum"))
    wdev = bt.repack_ternary(to_dev(bt.pack_ternary(c["w"]).reshape(-1), dev), n, k)
    need = bt.matmul_workspace_bytes(m, n, k)
    ws = torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device=dev) if need else None
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
    bt.ternary_matmul(xq, xs, xsum, wdev, n, c["w_scale"], y=y, acc=acc, workspace=ws)
    torch.cuda.synchronize()
    got_acc = acc.cpu().numpy()
    bad = np.argwhere(got_acc != ref["acc"])
    assert bad.size == 0, (len(bad), bad[:3])
    assert np.array_equal(y.cpu().numpy(), ref["y"])


def seeded_gemv_shapes(count=16, seed=2027):
    """M <= 16 (the GEMV), N and K drawn wide: tails in N, K a multiple of 128
    (not always of 256), K long enough to need a split for some M."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 17)), int(rng.integers(1, 20000)),
             128 * int(rng.integers(1, 81))) for _ in range(count)]


@pytest.mark.parametrize("m,n,k", seeded_gemv_shapes())
def test_gemv_seeded_shape(dev, m, n, k):
    c = synth.small_problem(78, m, n, k, "outlier")
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    xq, xs, xsum = (to_dev(ref[k_], dev) for k_ in ("q", "d", "qsum"))
    wdev = bt.repack_ternary(to_dev(bt.pack_ternary(c["w"]).reshape(-1), dev), n, k)
    need = bt.matmul_workspace_bytes(m, n, k)
    ws = torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device=dev) if need else None
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
    bt.ternary_matmul(xq, xs, xsum, wdev, n, c["w_scale"], y=y, acc=acc, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert np.array_equal(y.cpu().numpy(), ref["y"])


def seeded_int8_shapes(seed=2028):
    """I8_S: weight matrices small enough for the LDS-resident kernel (K <= 512)
    over many tokens, and general shapes with K a multiple of 32."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < 8:
        m, n, k = int(rng.integers(17, 60000)), int(rng.integers(16, 300)), 32 * int(rng.integers(1, 17))
        if m * n * k <= 1e9:
            out.append((m, n, k))
    while len(out) < 18:
        m, n, k = int(rng.integers(17, 3000)), int(rng.integers(17, 3000)), 32 * int(rng.integers(1, 257))
        if m * n * k <= 1.5e9:
            out.append((m, n, k))
    return out


@pytest.mark.parametrize("m,n,k", seeded_int8_shapes())
def test_int8_seeded_shape(dev, m, n, k):
    rng = np.random.default_rng(m + 7 * n + 13 * k)
    x = synth.small_problem(79, m, 16, max(k, 128), "t3")["x"][:, :k].copy()
    w8 = rng.integers(-128, 128, (n, k), dtype=np.int8)
    s = np.float32(rng.uniform(0.001, 0.01))
    ref = oracle.i8s_forward_ref(x, w8, s)
    xq, xs, _ = bt.quantize_act(to_dev(x, dev))
    w8dev = bt.repack_int8(to_dev(w8, dev))
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
    bt.int8_matmul(xq, xs, w8dev, n, s, y=y, acc=acc)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), ref["q"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert np.array_equal(y.cpu().numpy(), ref["y"])
