"""Grouped prefill GEMMs: many independent projections with M > 16 in one
persistent launch (a matmul plan whose descriptors all have M > 16), each
projection walking its own 128 x 256 output tiles on workgroup slots of its own;
a projection with few tiles and a long K is split into K ranges whose partial
sums a second launch adds.

Bar: the int32 accumulators equal the oracle's in every element, y within 1e-6
relative (exactly 0 where the oracle's is 0), and y equals the single-call
result of the same projection bit for bit (same arithmetic). Outputs are
poisoned before every launch.
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _rel(name, got, want):
    assert np.isfinite(got).all(), f"{name}: non-finite output (unwritten element?)"
    zero = want == 0
    assert (got[zero] == 0).all(), f"{name}: nonzero where the oracle is exactly 0"
    g, w = got[~zero].astype(np.float64), want[~zero].astype(np.float64)
    rel = np.abs(g - w) / np.abs(w)
    assert rel.size == 0 or rel.max() <= RTOL, f"{name}: max rel err {rel.max():.3e}"


def _problem(dev, case, with_acc):
    c = case
    n, k = c["w"].shape
    m = c["x"].shape[0]
    wdev = bt.repack_ternary(torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev), n, k)
    xq, xs, xsum = bt.quantize_act(torch.from_numpy(c["x"]).to(dev))
    it = {"xq": xq, "xscale": xs, "xsum": xsum, "wdev": wdev, "n": n, "w_scale": c["w_scale"],
          "y": torch.full((m, n), float("nan"), device=dev)}
    if with_acc:
        it["acc"] = torch.full((m, n), POISON_I32, dtype=torch.int32, device=dev)
    return it


def _check(dev, cases, items, plan, relaunches=1):
    for r in range(relaunches):
        for it in items:
            it["y"].fill_(float("nan"))
            if "acc" in it:
                it["acc"].fill_(POISON_I32)
        plan.launch()
        torch.cuda.synchronize()
        for i, (c, it) in enumerate(zip(cases, items)):
            m, n, k = c["x"].shape[0], c["w"].shape[0], c["w"].shape[1]
            tag = f"launch {r} projection {i} (M={m}, N={n}, K={k})"
            q = it["xq"].cpu().numpy()
            acc_ref = oracle.matmul_ref(q, c["w"], "f64")
            y = it["y"].cpu().numpy()
            _rel(f"{tag} y", y, oracle.dequant_ref(acc_ref, it["xscale"].cpu().numpy(),
                                                   c["w_scale"]))
            if "acc" in it:
                assert np.array_equal(it["acc"].cpu().numpy(), acc_ref), tag
            single = bt.ternary_matmul(it["xq"], it["xscale"], it["xsum"], it["wdev"], n,
                                       c["w_scale"], workspace=bt.new_workspace(m, n, k, dev))
            torch.cuda.synchronize()
            assert np.array_equal(single.cpu().numpy(), y), f"{tag}: differs from a single call"


def test_grouped_gemm_ragged_mixed_k(dev):
    """Ragged M, N and K (K not a multiple of 256), tiny and many-tile problems,
    different K in one launch, with and without accumulators, relaunched."""
    shapes = [(4133, 4100, 384), (17, 40, 128), (300, 2048, 1536), (129, 130, 1664),
              (1000, 1536, 8960), (2000, 512, 640), (33, 17920, 256)]
    cases = [synth.small_problem(70 + i, m, n, k, "t3", (0.3, 0.4, 0.3))
             for i, (m, n, k) in enumerate(shapes)]
    items = [_problem(dev, c, with_acc=(i % 2 == 0)) for i, c in enumerate(cases)]
    plan = bt.MatmulPlan(items)
    assert plan.workspace is not None   # (1000, 1536, 8960): 48 tiles, split along K
    _check(dev, cases, items, plan, relaunches=2)


def test_grouped_gemm_split_k(dev):
    """Projections with few output tiles and a long K are split into K ranges
    (ragged last range, odd stage counts, M just above 16, N not a multiple of
    the tile), beside unsplit ones; the ranges' partial sums are added by a
    second launch. Relaunched: the slices are rewritten and the zeros the
    ranges read as row sums stay zero."""
    shapes = [(300, 1000, 4480), (17, 40, 4224), (512, 1536, 8960), (129, 600, 1536),
              (40, 2048, 6144)]
    cases = [synth.small_problem(100 + i, m, n, k, "t3", (0.2, 0.6, 0.2))
             for i, (m, n, k) in enumerate(shapes)]
    items = [_problem(dev, c, with_acc=(i % 2 == 1)) for i, c in enumerate(cases)]
    plan = bt.MatmulPlan(items)
    assert plan.workspace is not None
    _check(dev, cases, items, plan, relaunches=2)


def test_grouped_gemm_many_ranges(dev):
    """The longest K the library takes, on one tile: 1024 stages in 64 ranges of
    16 (the reduce adds 64 slices, eight loads at a time), beside 8 ranges of a
    16384-wide K."""
    shapes = [(17, 40, 131072), (40, 60, 16384)]
    cases = [synth.small_problem(110 + i, m, n, k, "t3", (0.3, 0.4, 0.3))
             for i, (m, n, k) in enumerate(shapes)]
    items = [_problem(dev, c, with_acc=True) for c in cases]
    plan = bt.MatmulPlan(items)
    slices = [(m * n * 4 + 255) // 256 * 256 for m, n, _ in shapes]
    assert plan.workspace.numel() == 64 * slices[0] + 256 + 8 * slices[1] + 256
    _check(dev, cases, items, plan, relaunches=2)


def test_grouped_gemm_one_problem(dev):
    """A plan of one projection runs the same walk as the single persistent launch."""
    c = synth.small_problem(80, 4096, 4100, 512, "normal")
    items = [_problem(dev, c, with_acc=True)]
    _check(dev, [c], items, bt.MatmulPlan(items))


def test_grouped_gemm_decoder_layer_prefill(dev):
    """One decoder layer's four projections at M=512 (the one-layer prefill
    workload) in one launch, every output against the oracle."""
    cases = [synth.prefill_problem(p) for p in range(len(synth.PROJECTIONS))]
    items = [_problem(dev, c, with_acc=True) for c in cases]
    _check(dev, cases, items, bt.MatmulPlan(items))


def test_grouped_gemm_new_activations_in_same_buffers(dev):
    """A plan built once and launched again after new activations are quantized
    into its input buffers: the second launch reads the new inputs."""
    shapes = [(600, 2048, 1536), (600, 1536, 8960)]
    cases = [synth.small_problem(90 + i, m, n, k) for i, (m, n, k) in enumerate(shapes)]
    items = [_problem(dev, c, with_acc=True) for c in cases]
    plan = bt.MatmulPlan(items)
    _check(dev, cases, items, plan)
    for i, (c, it) in enumerate(zip(cases, items)):
        c2 = synth.small_problem(95 + i, *shapes[i], "t3")
        c["x"] = c2["x"]
        bt.quantize_act(torch.from_numpy(c2["x"]).to(dev), it["xq"], it["xscale"], it["xsum"])
    _check(dev, cases, items, plan)
