"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (from the method's definition: exact integer sums, then one fp32 rescale):
int8 q, fp32 d, int32 row sums and int32 accumulators bit-exact; fp32 y within
1e-6 relative (and exactly 0 where the oracle's y is 0). Every output buffer
is filled with NaN / an impossible integer before each call, so an element a
kernel forgets to write is caught (the blog post's NaN-at-batch-4/5 bug came
from a remainder path that left outputs unwritten).
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import ternary_weight_decoder_bt_amd as bt  # noqa: E402

RTOL = 1e-6
POISON_I32 = np.iinfo(np.int32).min   # |acc| <= 127*K never reaches it


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def assert_exact(name, got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches; first {i}: got {got[i]} want {want[i]}")


def assert_rel(name, got, want, rtol=RTOL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    assert np.isfinite(got).all(), f"{name}: non-finite output (unwritten element?)"
    zero = want == 0
    assert (got[zero] == 0).all(), f"{name}: nonzero where the oracle is exactly 0"
    rel = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    assert rel.size == 0 or rel.max() <= rtol, f"{name}: max rel err {rel.max():.3e}"


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def load_weights(w, dev):
    n, k = w.shape
    packed = to_dev(bt.pack_ternary(w).reshape(-1), dev)
    return bt.repack_ternary(packed, n, k)


def run_quantize(x, dev):
    m, k = x.shape
    xd = to_dev(x, dev)
    xq = torch.full((m, k), 99, dtype=torch.int8, device=dev)
    xs = torch.full((m,), float("nan"), dtype=torch.float32, device=dev)
    xsum = torch.full((m,), POISON_I32, dtype=torch.int32, device=dev)
    bt.quantize_act(xd, xq, xs, xsum)
    return xq, xs, xsum


def run_matmul(xq, xs, xsum, wdev, n, w_scale, dev, workspace=None):
    m = xq.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
    bt.ternary_matmul(xq, xs, xsum, wdev, n, w_scale, y=y, acc=acc, workspace=workspace)
    return y, acc


def check_full(case, dev, mode="f64", wdev=None):
    """The whole path on one projection, every output compared."""
    x, w, s = case["x"], case["w"], case["w_scale"]
    n = w.shape[0]
    ref = oracle.forward_ref(x, w, s, mode)
    xq, xs, xsum = run_quantize(x, dev)
    if wdev is None:
        wdev = load_weights(w, dev)
    y, acc = run_matmul(xq, xs, xsum, wdev, n, s, dev)
    torch.cuda.synchronize()
    assert_exact("q", xq.cpu().numpy(), ref["q"])
    assert_exact("d", xs.cpu().numpy(), ref["d"])
    assert_exact("qsum", xsum.cpu().numpy(), ref["qsum"])
    assert_exact("acc", acc.cpu().numpy(), ref["acc"])
    assert_rel("y", y.cpu().numpy(), ref["y"])
    return y, acc


# ------------------------------------------------------------------- repack

def test_grouped_repack_matches_single_and_oracle(dev):
    """One grouped launch gives every tensor the same bytes as its own repack
    (ragged N, K with a half 256-wide step, the decoder's shapes), twice in a
    row, and the grouped output drives the matmul to the oracle's result."""
    rng = np.random.default_rng(7)
    items, singles = [], []
    for n, k in [(2048, 1536), (40, 384), (17, 128), (1536, 8960), (33, 640)]:
        w = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
        packed = to_dev(bt.pack_ternary(w).reshape(-1), dev)
        singles.append(bt.repack_ternary(packed, n, k))
        out = torch.full((bt.repacked_bytes(n, k),), 0xAB, dtype=torch.uint8, device=dev)
        items.append((packed, n, k, out))
    plan = bt.RepackPlan(items)
    for _ in range(2):
        for *_, out in items:
            out.fill_(0xAB)
        plan.launch()
        torch.cuda.synchronize()
        for (_, n, k, out), single in zip(items, singles):
            assert torch.equal(out, single), (n, k)
    c = synth.small_problem(6, 5, 40, 384, "outlier")
    packed = to_dev(bt.pack_ternary(c["w"]).reshape(-1), dev)
    out = torch.empty(bt.repacked_bytes(40, 384), dtype=torch.uint8, device=dev)
    bt.RepackPlan([(packed, 40, 384, out)]).launch()
    check_full(c, dev, wdev=out)


# ------------------------------------------------------------ quantization

def test_quantize_single_gemv_input(dev):
    x = synth.config0()["x"]
    q, d, s = oracle.quantize_ref(x)
    xq, xs, xsum = run_quantize(x, dev)
    assert_exact("q", xq.cpu().numpy(), q)
    assert_exact("d", xs.cpu().numpy(), d)
    assert_exact("qsum", xsum.cpu().numpy(), s)


@pytest.mark.parametrize("m,k,dist", [(1, 8960, "outlier"), (7, 1536, "t3"), (64, 129, "normal"),
                                      (3, 20000, "t3"), (5, 6, "normal"), (300, 1536, "outlier")])
def test_quantize_shapes(dev, m, k, dist):
    rng = np.random.default_rng(m * 7 + k)
    x = {"normal": lambda: rng.standard_normal((m, k), dtype=np.float32),
         "t3": lambda: rng.standard_t(3, (m, k)).astype(np.float32),
         "outlier": lambda: rng.standard_normal((m, k), dtype=np.float32) *
         np.where(rng.random((m, k)) < 0.001, np.float32(20), np.float32(1))}[dist]()
    q, d, s = oracle.quantize_ref(x)
    xq, xs, xsum = run_quantize(x, dev)
    assert_exact("q", xq.cpu().numpy(), q)
    assert_exact("d", xs.cpu().numpy(), d)
    assert_exact("qsum", xsum.cpu().numpy(), s)


def test_quantize_long_prefill_rows(dev):
    for proj in (0, 3):
        x = synth.long_prefill_problem(0, proj, with_weights=False)["x"]
        q, d, s = oracle.quantize_ref(x)
        xq, xs, xsum = run_quantize(x, dev)
        assert_exact(f"q[{proj}]", xq.cpu().numpy(), q)
        assert_exact(f"d[{proj}]", xs.cpu().numpy(), d)
        assert_exact(f"qsum[{proj}]", xsum.cpu().numpy(), s)


def test_quantize_golden_ties(dev, golden):
    rows = golden("quantize_worked.txt")
    xs = {r[0]: [np.float32(v) for v in r[2:]] for r in rows if r[1] == "x"}
    qs = {r[0]: [int(v) for v in r[2:]] for r in rows if r[1] == "q"}
    labels = sorted(xs)
    for width in (6, 8, 128):        # scalar path, vector path, vector path with padding
        x = np.zeros((len(labels), width), np.float32)
        want = np.zeros((len(labels), width), np.int8)
        for i, l in enumerate(labels):
            x[i, :6] = xs[l]
            want[i, :6] = qs[l]
        xq, _, _ = run_quantize(x, dev)
        assert_exact(f"q(width {width})", xq.cpu().numpy(), want)


def test_quantize_tiny_and_zero_rows(dev):
    x = np.zeros((5, 256), np.float32)
    x[0, 5] = np.float32(1e-39)
    x[1, 6] = np.float32(-1e-37)
    x[2, 7], x[2, 8] = np.float32(1e-36), np.float32(-5e-37)
    x[4] = np.random.default_rng(1).standard_normal(256).astype(np.float32)
    q, d, s = oracle.quantize_ref(x)
    assert 0 < d[2] < np.finfo(np.float32).tiny
    xq, xs, xsum = run_quantize(x, dev)
    assert_exact("q", xq.cpu().numpy(), q)
    assert_exact("d", xs.cpu().numpy(), d)
    assert_exact("qsum", xsum.cpu().numpy(), s)


def test_grouped_quantize_mixed_rows(dev):
    """One grouped quantization launch over problems that take each of its paths:
    short rows four to a workgroup (K % 4 == 0, K <= 2048, with a ragged last
    workgroup), long rows one to a workgroup (K > 2048, K up to 9216 in registers
    and beyond), rows whose K is not a multiple of 4, tiny rows and a zero row.
    Relaunched with new activations in the same buffers."""
    shapes = [(5, 1536), (3, 100), (17, 2048), (2, 2052), (9, 8960), (1, 7), (4, 9220),
              (6, 4)]
    rng = np.random.default_rng(12)
    xs = [rng.standard_t(3, size=s).astype(np.float32) for s in shapes]
    xs[2][3] = 0.0
    dx = [to_dev(x, dev) for x in xs]
    outs = [(torch.full(s, 99, dtype=torch.int8, device=dev),
             torch.full((s[0],), float("nan"), dtype=torch.float32, device=dev),
             torch.full((s[0],), POISON_I32, dtype=torch.int32, device=dev)) for s in shapes]
    plan = bt.QuantPlan([(x,) + o for x, o in zip(dx, outs)])
    for rep in range(2):
        if rep:
            for x, d in zip(xs, dx):
                x[...] = rng.standard_normal(x.shape).astype(np.float32)
                d.copy_(torch.from_numpy(x))
            for o in outs:
                o[0].fill_(99)
                o[1].fill_(float("nan"))
        plan.launch()
        torch.cuda.synchronize()
        for i, (x, (xq, xsc, xsum)) in enumerate(zip(xs, outs)):
            q, d, s = oracle.quantize_ref(x)
            assert_exact(f"q[{i}]", xq.cpu().numpy(), q)
            assert_exact(f"d[{i}]", xsc.cpu().numpy(), d)
            assert_exact(f"qsum[{i}]", xsum.cpu().numpy(), s)


# ----------------------------------------------------------------- matmul

def test_single_gemv_workload(dev):
    check_full(synth.config0(), dev, mode="int64")


@pytest.mark.parametrize("m", list(range(1, 17)))
def test_gemv_every_m_ragged(dev, m):
    # N = 40 leaves a partial 16-row tile; K = 384 ends with a 128-wide step
    check_full(synth.small_problem(2, m, 40, 384), dev, mode="loops" if m <= 2 else "int64")


@pytest.mark.parametrize("m,n,k", [(1, 40, 1536), (5, 1536, 1536), (16, 1536, 8960),
                                   (3, 17, 128), (1, 1, 128), (8, 2048, 1664)])
def test_gemv_split_k_and_edges(dev, m, n, k):
    check_full(synth.small_problem(3, m, n, k, "outlier"), dev)


# Single calls with few 16-row tiles split each tile's K range over 2 or 4 waves
# of a workgroup: 5 steps over 4 waves leaves one wave empty, 1152 and 640 end
# in a 128-wide step, 625 tiles take 2 waves each, and 16 x 8960 also splits K
# across workgroups.
@pytest.mark.parametrize("m,n,k", [(1, 40, 1280), (3, 1000, 1152), (2, 33, 768),
                                   (16, 10000, 640), (16, 1536, 8960), (5, 17, 1280)])
@pytest.mark.parametrize("fused", [False, True])
def test_gemv_wave_split_k(dev, m, n, k, fused):
    c = synth.small_problem(31, m, n, k, "outlier")
    if fused:
        ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
        y, acc, _ = run_fused(c, dev)
        assert_exact("acc", acc.cpu().numpy(), ref["acc"])
        assert_rel("y", y.cpu().numpy(), ref["y"])
    else:
        check_full(c, dev)


# Single calls on quantized rows that still have few workgroups split each
# tile's 16 weight rows over two workgroups, each loading and storing its own 8:
# N = 8 leaves the second half of the only tile empty, N = 9 one valid row in
# it, N = 24 half a tile at the end; the down (8960 -> 1536) and qkv
# (1536 -> 2048) shapes run split too, and K = 8960 also splits each tile's K
# range over the waves of its workgroup.
@pytest.mark.parametrize("m,n,k", [(1, 8, 8960), (3, 9, 8960), (2, 24, 1536),
                                   (1, 1536, 8960), (3, 2048, 1536)])
def test_gemv_row_parts(dev, m, n, k):
    check_full(synth.small_problem(37, m, n, k, "outlier"), dev)


_REMAINDER_W = {}


@pytest.mark.parametrize("proj", ["gate_up", "down"])
@pytest.mark.parametrize("m", synth.REMAINDER_MS)
def test_decode_remainder_sweep(dev, proj, m):
    c = synth.decode_remainder_problem(proj, m)
    key = proj
    if key not in _REMAINDER_W:
        _REMAINDER_W.clear()
        _REMAINDER_W[key] = load_weights(c["w"], dev)
    check_full(c, dev, wdev=_REMAINDER_W[key])


# (40, 60, 16384): one 64 x 64 tile, K split into 16 ranges, so the reduce launch
# adds its slices in two rounds of (up to) eight loads
@pytest.mark.parametrize("m,n,k", [(17, 40, 384), (33, 200, 128), (100, 2048, 1536),
                                   (128, 128, 256), (129, 130, 1664), (300, 1536, 8960),
                                   (40, 60, 16384)])
def test_gemm_shapes(dev, m, n, k):
    check_full(synth.small_problem(4, m, n, k, "t3", (0.3, 0.4, 0.3)), dev)


# Shapes with enough output tiles for the persistent GEMM (several tiles per
# workgroup, pipeline crossing tile boundaries), with ragged M, N a multiple
# of 4 but not of the tile, N not a multiple of 4, and stage counts that are
# and are not a multiple of the pipeline depth. Every output is compared.
# (4000, 1530, 640): 128 x 96 tiles (512 of them against 384 of 128 x 128), ragged M, N, K;
# (2000, 2000, 640): 128 x 128 tiles (256, one per compute unit), ragged M, N, K
@pytest.mark.parametrize("m,n,k", [(4133, 4100, 384), (4100, 4099, 256), (4096, 8192, 640),
                                   (4000, 1530, 640), (2000, 2000, 640)])
def test_gemm_many_tiles_ragged(dev, m, n, k):
    check_full(synth.small_problem(5, m, n, k, "t3", (0.3, 0.4, 0.3)), dev)


@pytest.mark.parametrize("proj", [0, 1, 2, 3])
def test_prefill_one_layer(dev, proj):
    check_full(synth.prefill_problem(proj), dev)


@pytest.mark.parametrize("layer,proj", [(0, 0), (0, 1), (0, 2), (0, 3), (27, 3)])
def test_long_prefill_sampled(dev, layer, proj):
    c = synth.long_prefill_problem(layer, proj)
    x, w, s = c["x"], c["w"], c["w_scale"]
    m, n = x.shape[0], w.shape[0]
    q, d, qs = oracle.quantize_ref(x)
    xq, xs, xsum = run_quantize(x, dev)
    y, acc = run_matmul(xq, xs, xsum, load_weights(w, dev), n, s, dev)
    torch.cuda.synchronize()
    assert_exact("q", xq.cpu().numpy(), q)
    assert_exact("d", xs.cpu().numpy(), d)
    y, acc = y.cpu().numpy(), acc.cpu().numpy()
    rng = np.random.default_rng(layer * 10 + proj)
    rows = np.unique(np.r_[0, 1, 127, 128, m - 1, rng.integers(0, m, 6)])
    cols = np.unique(np.r_[0, 15, 16, n - 1, rng.integers(0, n, 6)])
    acc_rows = oracle.matmul_ref(q[rows], w, "f64")
    acc_cols = oracle.matmul_ref(q, w[cols], "f64")
    assert_exact("acc rows", acc[rows], acc_rows)
    assert_exact("acc cols", acc[:, cols], acc_cols)
    assert_rel("y rows", y[rows], oracle.dequant_ref(acc_rows, d[rows], s))
    assert_rel("y cols", y[:, cols], oracle.dequant_ref(acc_cols, d, s))
    assert np.isfinite(y).all() and (acc != POISON_I32).all()


def test_worst_case_accumulator(dev):
    k = 8960
    for m in (1, 32):
        x = np.ones((m, k), np.float32)
        w = np.ones((32, k), np.int8)
        w[16:] = -1
        y, acc = check_full({"x": x, "w": w, "w_scale": np.float32(0.5)}, dev)
        a = acc.cpu().numpy()
        assert (a[:, :16] == 1_137_920).all() and (a[:, 16:] == -1_137_920).all()


@pytest.mark.parametrize("m", [1, 4, 16, 48])
def test_layout_identity_and_one_hot(dev, m):
    rng = np.random.default_rng(m)
    k = 256
    x = rng.standard_normal((m, k), dtype=np.float32)
    q, _, _ = oracle.quantize_ref(x)
    xq, xs, xsum = run_quantize(x, dev)
    _, acc = run_matmul(xq, xs, xsum, load_weights(np.eye(k, dtype=np.int8), dev), k, 1.0, dev)
    assert_exact("identity", acc.cpu().numpy(), q.astype(np.int32))
    kstar = rng.integers(0, k, 48)
    w = np.zeros((48, k), np.int8)
    w[np.arange(48), kstar] = 1
    _, acc = run_matmul(xq, xs, xsum, load_weights(w, dev), 48, 1.0, dev)
    assert_exact("one-hot", acc.cpu().numpy(), q[:, kstar].astype(np.int32))


def test_zero_row_in_batch_gives_zero_output(dev):
    for m in (4, 20):
        c = synth.small_problem(5, m, 64, 256)
        c["x"][1] = 0
        y, _ = check_full(c, dev)
        assert (y.cpu().numpy()[1] == 0).all()


def test_split_gemv_deterministic_with_poisoned_workspace(dev):
    """M = 16 rows of K = 8960 do not fit one LDS slice, so K is split: the
    chunks' partial sums go to workspace slices and a second launch adds them.
    Two calls agree bit for bit with the oracle whatever the workspace held."""
    c = synth.small_problem(6, 16, 1536, 8960)
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    wdev = load_weights(c["w"], dev)
    xq, xs, xsum = run_quantize(c["x"], dev)
    ws = bt.new_workspace(16, 1536, 8960, dev)
    assert ws is not None
    for fill in (0x00, 0x7F):
        ws.fill_(fill)
        y, a = run_matmul(xq, xs, xsum, wdev, 1536, c["w_scale"], dev, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy(), ref["acc"])
        assert np.array_equal(y.cpu().numpy(), ref["y"])
    # the fused path splits the same way and keeps its scales in the workspace
    for keep in (True, False):
        ws.fill_(0x3C)
        out = {}
        if keep:
            out = dict(xq=torch.empty_like(xq), xscale=torch.empty_like(xs),
                       xsum=torch.empty_like(xsum))
        y, a = bt.ternary_matmul_fused(to_dev(c["x"], dev), wdev, 1536, c["w_scale"],
                                       workspace=ws, want_acc=True, **out)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy(), ref["acc"])
        assert np.array_equal(y.cpu().numpy(), ref["y"])
        if keep:
            assert np.array_equal(out["xscale"].cpu().numpy(), ref["d"])
            assert np.array_equal(out["xsum"].cpu().numpy(), ref["qsum"])


# ------------------------------------------------------------------ grouped

def test_grouped_decode_layers(dev):
    items_q, items_m, refs = [], [], []
    for layer in (0, 27):
        for proj in range(4):
            c = synth.decode_problem(layer, proj)
            m, k, n = c["M"], c["K"], c["N"]
            x = to_dev(c["x"], dev)
            xq = torch.full((m, k), 99, dtype=torch.int8, device=dev)
            xs = torch.full((m,), float("nan"), dtype=torch.float32, device=dev)
            xsum = torch.full((m,), POISON_I32, dtype=torch.int32, device=dev)
            y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
            acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
            items_q.append((x, xq, xs, xsum))
            items_m.append({"xq": xq, "xscale": xs, "xsum": xsum, "wdev": load_weights(c["w"], dev),
                            "n": n, "w_scale": c["w_scale"], "y": y, "acc": acc})
            refs.append(oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64"))
    qp, mp = bt.QuantPlan(items_q), bt.MatmulPlan(items_m)
    for rep in range(2):
        qp.launch()
        mp.launch()
        torch.cuda.synchronize()
        for i, (it, ref) in enumerate(zip(items_m, refs)):
            assert_exact(f"q[{i}]", it["xq"].cpu().numpy(), ref["q"])
            assert_exact(f"acc[{i}]", it["acc"].cpu().numpy(), ref["acc"])
            assert_rel(f"y[{i}]", it["y"].cpu().numpy(), ref["y"])


# ------------------------------------------------------- fused quantization

def run_fused(c, dev, with_outputs=True, wdev=None):
    x, w, s = c["x"], c["w"], c["w_scale"]
    m, k = x.shape
    n = w.shape[0]
    if wdev is None:
        wdev = load_weights(w, dev)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
    outs = (None, None, None)
    if with_outputs:
        outs = (torch.full((m, k), 99, dtype=torch.int8, device=dev),
                torch.full((m,), float("nan"), dtype=torch.float32, device=dev),
                torch.full((m,), POISON_I32, dtype=torch.int32, device=dev))
    bt.ternary_matmul_fused(to_dev(x, dev), wdev, n, s, y=y, acc=acc, xq=outs[0], xscale=outs[1],
                            xsum=outs[2])
    torch.cuda.synchronize()
    return y, acc, outs


@pytest.mark.parametrize("m,n,k", [(1, 1536, 1536), (1, 40, 384), (3, 17920, 1536),
                                   (4, 1536, 8960), (16, 200, 640), (2, 1, 128), (7, 2048, 8960)])
def test_fused_quantize_gemv(dev, m, n, k):
    c = synth.small_problem(7, m, n, k, "outlier")
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    y, acc, (xq, xs, xsum) = run_fused(c, dev)
    assert_exact("q", xq.cpu().numpy(), ref["q"])
    assert_exact("d", xs.cpu().numpy(), ref["d"])
    assert_exact("qsum", xsum.cpu().numpy(), ref["qsum"])
    assert_exact("acc", acc.cpu().numpy(), ref["acc"])
    assert_rel("y", y.cpu().numpy(), ref["y"])


def test_fused_without_optional_outputs_and_zero_rows(dev):
    c = synth.small_problem(8, 5, 300, 1536, "t3")
    c["x"][2] = 0
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    y, acc, _ = run_fused(c, dev, with_outputs=False)
    assert_exact("acc", acc.cpu().numpy(), ref["acc"])
    assert_rel("y", y.cpu().numpy(), ref["y"])
    assert (y.cpu().numpy()[2] == 0).all()


def _grouped_items(cases, dev, fused):
    items, refs = [], []
    for c in cases:
        m, k = c["x"].shape
        n = c["w"].shape[0]
        it = {"wdev": load_weights(c["w"], dev), "n": n, "w_scale": c["w_scale"],
              "y": torch.full((m, n), float("nan"), dtype=torch.float32, device=dev),
              "acc": torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev),
              "xq": torch.full((m, k), 99, dtype=torch.int8, device=dev),
              "xscale": torch.full((m,), float("nan"), dtype=torch.float32, device=dev),
              "xsum": torch.full((m,), POISON_I32, dtype=torch.int32, device=dev)}
        if fused:
            it["x"] = to_dev(c["x"], dev)
        else:
            bt.quantize_act(to_dev(c["x"], dev), it["xq"], it["xscale"], it["xsum"])
        items.append(it)
        refs.append(oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64"))
    return items, refs


def _check_grouped(items, refs):
    for i, (it, ref) in enumerate(zip(items, refs)):
        assert_exact(f"q[{i}]", it["xq"].cpu().numpy(), ref["q"])
        assert_exact(f"d[{i}]", it["xscale"].cpu().numpy(), ref["d"])
        assert_exact(f"qsum[{i}]", it["xsum"].cpu().numpy(), ref["qsum"])
        assert_exact(f"acc[{i}]", it["acc"].cpu().numpy(), ref["acc"])
        assert_rel(f"y[{i}]", it["y"].cpu().numpy(), ref["y"])


@pytest.mark.parametrize("fused", [False, True])
def test_grouped_fused_decode_layers(dev, fused):
    cases = [synth.decode_problem(layer, proj) for layer in (0, 13) for proj in range(4)]
    items, refs = _grouped_items(cases, dev, fused)
    plan = bt.MatmulPlan(items)
    for _ in range(2):
        plan.launch()
        torch.cuda.synchronize()
        _check_grouped(items, refs)


@pytest.mark.parametrize("fused", [False, True])
def test_grouped_new_activations_each_launch(dev, fused):
    """How a decoder uses a plan: built once, then each step writes new
    activations into the same buffers and launches it again. Four launches,
    every output poisoned before each and checked against the oracle for that
    step's rows; the third step's first projection gets an all-zero row (d = 0,
    q = 0) between live ones, so no launch may lean on what an earlier one left."""
    cases = [synth.decode_problem(layer, proj, m) for layer, m in ((0, 1), (27, 3))
             for proj in range(4)]
    items, _ = _grouped_items(cases, dev, fused)
    plan = bt.MatmulPlan(items)
    for step in range(4):
        refs = []
        for i, (c, it) in enumerate(zip(cases, items)):
            m, k = c["x"].shape
            rng = np.random.default_rng(1000 * step + i)
            x = rng.standard_normal((m, k)).astype(np.float32)
            if step == 2 and i == 0:
                x[0] = 0.0
            it["y"].fill_(float("nan"))
            it["acc"].fill_(POISON_I32)
            if fused:
                it["x"].copy_(to_dev(x, dev))
                it["xq"].fill_(99)
                it["xscale"].fill_(float("nan"))
                it["xsum"].fill_(POISON_I32)
            else:
                bt.quantize_act(to_dev(x, dev), it["xq"], it["xscale"], it["xsum"])
            refs.append(oracle.forward_ref(x, c["w"], c["w_scale"], "f64"))
        plan.launch()
        torch.cuda.synchronize()
        _check_grouped(items, refs)


@pytest.mark.parametrize("fused", [False, True])
def test_grouped_mixed_m_with_lds_split(dev, fused):
    # M = 16 rows of K = 8960 do not fit one LDS slice, so that projection is
    # split along K inside the grouped launch and uses the plan's workspace
    cases = [synth.small_problem(9, 16, 1536, 8960), synth.small_problem(9, 1, 2048, 1536),
             synth.small_problem(9, 3, 40, 384, "t3"), synth.small_problem(9, 5, 17920, 1536)]
    items, refs = _grouped_items(cases, dev, fused)
    plan = bt.MatmulPlan(items)
    assert plan.workspace is not None
    for _ in range(3):
        for it in items:
            it["y"].fill_(float("nan"))
        plan.launch()
        torch.cuda.synchronize()
        _check_grouped(items, refs)
    assert int(plan.workspace.count_nonzero()) == 0


@pytest.mark.parametrize("fused", [False, True])
def test_grouped_batched_decode_split_repeated(dev, fused):
    """A 16-token batch through four layers' projections in one plan: every
    down projection (16 x 8960 activations) is split over K ranges whose
    partial sums meet through atomics, the last range to arrive finishing the
    tile. Thirty launches in a row, each checked exactly (acc, q) and within
    the tolerance (y) against the oracle, and the workspace left clean: an
    ordering mistake between a range's additions and its arrival count would
    show as a wrong sum in some launch."""
    cases = [synth.decode_problem(layer, proj, 16) for layer in (0, 5, 11, 27)
             for proj in range(4)]
    items, refs = _grouped_items(cases, dev, fused)
    plan = bt.MatmulPlan(items)
    assert plan.workspace is not None
    down = [i for i, c in enumerate(cases) if c["K"] == 8960]
    for rep in range(30):
        for i in down:
            items[i]["y"].fill_(float("nan"))
            items[i]["acc"].fill_(POISON_I32)
        plan.launch()
        torch.cuda.synchronize()
        for i in down:
            assert_exact(f"acc[{i}] launch {rep}", items[i]["acc"].cpu().numpy(), refs[i]["acc"])
            assert_rel(f"y[{i}] launch {rep}", items[i]["y"].cpu().numpy(), refs[i]["y"])
    _check_grouped(items, refs)
    assert int(plan.workspace.count_nonzero()) == 0


# 64 x 64 tiles in 3, 3, 2 and 2 ranges; (1500, 1530, 8960): 128 x 96 tiles in 2 ranges;
# (1700, 1900, 8960): 128 x 128 tiles in 2 ranges
@pytest.mark.parametrize("m,n,k", [(150, 1536, 8960), (130, 1540, 8960), (17, 130, 2048),
                                   (512, 1536, 8960), (1500, 1530, 8960), (1700, 1900, 8960)])
def test_gemm_split_k_exact_and_workspace_clean(dev, m, n, k):
    """Few output tiles and a long K: K is split and the int32 partial sums meet
    in the workspace; the result is the oracle's, bit for bit, on two calls in a
    row with the same workspace (poisoned in between: every slice is rewritten)."""
    need = bt.matmul_workspace_bytes(m, n, k)
    assert need > 0
    c = synth.small_problem(60, m, n, k, "t3", (0.2, 0.6, 0.2))
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    wdev = load_weights(c["w"], dev)
    xq, xs, xsum = (to_dev(ref[k_], dev) for k_ in ("q", "d", "qsum"))
    for _ in range(2):
        y, acc = run_matmul(xq, xs, xsum, wdev, n, c["w_scale"], dev, workspace=ws)
        torch.cuda.synchronize()
        assert_exact("acc", acc.cpu().numpy(), ref["acc"])
        assert np.array_equal(y.cpu().numpy(), ref["y"])
        ws.fill_(0x5A)


# ------------------------------------------------------ the longest K taken
#
# K = BT_MAX_K = 131072 on every path: single GEMV unfused (M = 1, 5; K split
# into workgroup ranges whose slices a reduce launch adds) and fused (the row
# read twice), GEMM (M = 17, 300: K split into many ranges), random operands
# against the oracle, and the largest accumulator the bound allows: every q =
# 127 and every weight +1 gives acc = 127 * 131072 = 16,646,144 < 2^24, exact in
# int32 and in fp32.
@pytest.mark.parametrize("m", [1, 5, 17, 300])
def test_maximum_k_every_path(dev, m):
    k, n = 131072, 40
    check_full(synth.small_problem(120 + m, m, n, k, "outlier", (0.3, 0.4, 0.3)), dev)
    x = np.full((m, k), 0.75, np.float32)
    w = np.ones((n, k), np.int8)
    ref = oracle.forward_ref(x, w, np.float32(0.5), "int64")
    assert int(ref["acc"].max()) == 127 * k
    y, acc = check_full({"x": x, "w": w, "w_scale": np.float32(0.5)}, dev, mode="int64")
    assert int(acc.max().item()) == 127 * k
    if m <= 16:
        c = synth.small_problem(130 + m, m, n, k, "t3")
        ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
        wdev = load_weights(c["w"], dev)
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
        acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
        bt.ternary_matmul_fused(to_dev(c["x"], dev), wdev, n, c["w_scale"], y=y, acc=acc)
        torch.cuda.synchronize()
        assert_exact("fused acc", acc.cpu().numpy(), ref["acc"])
        assert_rel("fused y", y.cpu().numpy(), ref["y"])


# ------------------------------------------------------------ degenerate cases
#
# One output row on the GEMM path, one 128-element group, all-zero weights (the
# code offset then cancels exactly: every code is 1, so sum q*c - sum q = 0 and y
# is exactly 0), and the GEMV / GEMM boundary: rows 0..15 of an M = 17 GEMM
# equal the M = 16 GEMV of the same rows bit for bit.
@pytest.mark.parametrize("m,n,k", [(17, 1, 128), (300, 1, 1536), (1, 7, 128), (40, 300, 128)])
def test_degenerate_shapes(dev, m, n, k):
    check_full(synth.small_problem(140, m, n, k, "t3"), dev, mode="int64")


@pytest.mark.parametrize("m", [1, 16, 17, 512])
def test_all_zero_weights(dev, m):
    c = synth.small_problem(141, m, 100, 1536, "outlier", (0.0, 1.0, 0.0))
    assert not c["w"].any()
    y, acc = check_full(c, dev, mode="int64")
    assert not acc.any().item() and not y.any().item()


def test_gemv_gemm_boundary_agree(dev):
    c = synth.small_problem(142, 17, 1536, 8960, "outlier")
    wdev = load_weights(c["w"], dev)
    y17, acc17 = check_full(c, dev, wdev=wdev)
    c16 = dict(c, x=c["x"][:16])
    y16, acc16 = check_full(c16, dev, wdev=wdev)
    assert torch.equal(acc16, acc17[:16])
    assert torch.equal(y16, y17[:16])
