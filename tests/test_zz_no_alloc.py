"""The allocation-free entry point (bt_ternary_matmul_noalloc) against
bt_ternary_matmul with a caller-owned workspace: same arguments, the split-K
partial sums in the library's own device array instead.

Bar: int32 accumulators bit-exact, y within 1e-6 relative (exactly 0 where the
reference is 0), and both against the oracle's q / acc. Each case makes two
calls in a row on one stream, the second with a smaller input, so the second
runs on whatever the first left in the shared array.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import ternary_weight_decoder_bt_amd as bt  # noqa: E402

RTOL = 1e-6
POISON_I32 = np.iinfo(np.int32).min
LIMIT = 16 << 20


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _rel(name, got, want):
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    zero = want == 0
    assert (got[zero] == 0).all(), f"{name}: nonzero where the reference is 0"
    g, w = got[~zero].astype(np.float64), want[~zero].astype(np.float64)
    rel = np.abs(g - w) / np.abs(w)
    assert rel.size == 0 or rel.max() <= RTOL, f"{name}: max rel err {rel.max():.3e}"


def _prepare(dev, seed, m, n, k):
    c = synth.small_problem(seed, m, n, k, "t3", (0.3, 0.4, 0.3))
    w = c["w"]
    wdev = bt.repack_ternary(torch.from_numpy(bt.pack_ternary(w).reshape(-1)).to(dev), n, k)
    xq, xs, xsum = bt.quantize_act(torch.from_numpy(c["x"]).to(dev))
    return c, wdev, (xq, xs, xsum)


# (first call, second smaller call): split-K GEMVs (K = 8960 does not fit one
# LDS slice at these token counts), split-K GEMMs, and shapes with no split
CASES = [
    ((16, 1536, 8960), (8, 1536, 8960)),
    ((512, 1536, 8960), (150, 1536, 8960)),
    ((300, 2048, 8960), (40, 640, 4096)),
    ((1, 1536, 1536), (1, 256, 128)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_entry_point(dev, first, second):
    runs = []
    for seed, (m, n, k) in enumerate((first, second)):
        print(f"noalloc case M={m} N={n} K={k}", flush=True)
        need = bt.matmul_workspace_bytes(m, n, k)
        assert need <= LIMIT
        c, wdev, q = _prepare(dev, 40 + seed, m, n, k)
        ws = bt.new_workspace(m, n, k, dev)
        y_ref = torch.full((m, n), float("nan"), device=dev)
        acc_ref = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
        bt.ternary_matmul(*q, wdev, n, c["w_scale"], y=y_ref, acc=acc_ref, workspace=ws)
        y = torch.full((m, n), float("nan"), device=dev)
        acc = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
        y2 = torch.full((m, n), float("nan"), device=dev)
        runs.append((c, q, y_ref, acc_ref, y, acc, y2, wdev, need))
    # the two shapes back to back on one stream, each with and without acc
    for c, q, _, _, y, acc, y2, wdev, _ in runs:
        n = y.shape[1]
        bt.ternary_matmul_noalloc(*q, wdev, n, c["w_scale"], y, acc)
        bt.ternary_matmul_noalloc(*q, wdev, n, c["w_scale"], y2)
    torch.cuda.synchronize()
    for c, q, y_ref, acc_ref, y, acc, y2, _, need in runs:
        tag = f"M={y.shape[0]} N={y.shape[1]} K={c['K']} scratch={need}"
        qn = q[0].cpu().numpy()
        want_acc = oracle.matmul_ref(qn, c["w"], "f64")
        assert np.array_equal(acc_ref.cpu().numpy(), want_acc), tag
        assert np.array_equal(acc.cpu().numpy(), acc_ref.cpu().numpy()), tag
        _rel(f"{tag} y", y.cpu().numpy(), y_ref.cpu().numpy())
        _rel(f"{tag} y without acc", y2.cpu().numpy(), y_ref.cpu().numpy())
        _rel(f"{tag} y vs oracle", y.cpu().numpy(),
             oracle.dequant_ref(want_acc, q[1].cpu().numpy(), c["w_scale"]))


def test_noalloc_repeated_calls_agree(dev):
    """Ten calls alternating a large and a small split shape: every output of
    every call equals the workspace entry point's."""
    shapes = [(512, 1536, 8960), (16, 1536, 8960)]
    prepared = []
    for seed, (m, n, k) in enumerate(shapes):
        c, wdev, q = _prepare(dev, 60 + seed, m, n, k)
        y_ref = bt.ternary_matmul(*q, wdev, n, c["w_scale"],
                                  workspace=bt.new_workspace(m, n, k, dev))
        prepared.append((c, wdev, q, y_ref))
    outs = []
    for i in range(10):
        c, wdev, q, _ = prepared[i % 2]
        n = c["N"]
        y = torch.full((c["M"], n), float("nan"), device=dev)
        bt.ternary_matmul_noalloc(*q, wdev, n, c["w_scale"], y)
        outs.append((i % 2, y))
    torch.cuda.synchronize()
    for j, y in outs:
        assert torch.equal(y, prepared[j][3])


def test_noalloc_rejects_oversized_split(dev):
    m, n, k = 2054, 1024, 8960
    assert bt.matmul_workspace_bytes(m, n, k) > LIMIT
    xq = torch.zeros((m, k), dtype=torch.int8, device=dev)
    xs = torch.zeros(m, dtype=torch.float32, device=dev)
    xsum = torch.zeros(m, dtype=torch.int32, device=dev)
    wdev = torch.zeros(bt.repacked_bytes(n, k), dtype=torch.uint8, device=dev)
    y = torch.full((m, n), 7.0, device=dev)
    with pytest.raises(bt.BtError, match="BT_ERR_WORKSPACE"):
        bt.ternary_matmul_noalloc(xq, xs, xsum, wdev, n, 0.5, y)
    torch.cuda.synchronize()
    assert (y == 7.0).all()
