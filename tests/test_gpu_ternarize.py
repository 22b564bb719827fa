"""GPU parity for the offline ternarization (bt_ternarize) through the C ABI
against the CPU oracle (oracle/bitnet_ref.py): the packed bytes bit-exact and
the per-tensor scale gamma bit-exact, on the hand-worked example with ties,
on seeded weights shaped like the decoder's projections (normal, outliers,
Student-t), on an all-zero tensor and on one full gate_up tensor; then the
ternarized weights feed the matmul.

Source: "VibeVoice-ASR-BitNet Technical Report" section 2.2.2 (ternary weights
following its BitNet reference's absmean quantizer).
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import ternary_weight_decoder_bt_amd as bt  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run(w, eps, dev, poison=True):
    wd = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    n, k = w.shape
    packed = torch.full((n * k // 4,), 0xFF, dtype=torch.uint8, device=dev)  # code 3 everywhere
    scale = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(bt.ternarize_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    if poison:
        ws.fill_(0x7F)
    bt.ternarize(wd, eps, packed=packed, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return packed.cpu().numpy().reshape(n, k // 4), np.float32(scale.cpu().numpy()[0])


def check(w, eps, dev):
    want_p, want_g = oracle.ternarize_pack_ref(w, eps)
    got_p, got_g = run(w, eps, dev)
    assert got_g.view(np.uint32) == want_g.view(np.uint32), (float(got_g), float(want_g))
    if not np.array_equal(got_p, want_p):
        bad = np.argwhere(got_p != want_p)
        raise AssertionError(f"{len(bad)} packed bytes differ; first {bad[:4].tolist()}")


def test_hand_worked_golden(dev, golden):
    vals, c0, c25 = [], [], []
    for v, count, a, b in golden("ternarize_worked.txt"):
        vals += [float(v)] * int(count)
        c0 += [int(a)] * int(count)
        c25 += [int(b)] * int(count)
    w = np.array(vals, np.float32).reshape(2, 128)
    for eps, codes in ((0.0, c0), (0.25, c25)):
        got_p, got_g = run(w, eps, dev)
        assert got_g == np.float32(0.25)
        np.testing.assert_array_equal(bt.unpack_ternary(got_p, 128),
                                      np.array(codes, np.int8).reshape(2, 128))


@pytest.mark.parametrize("n,k,dist,eps", [
    (1536, 1536, "normal", 0.0), (2048, 1536, "outlier", 1e-5), (1536, 8960, "t3", 0.0),
    (17, 128, "normal", 1e-3), (1, 384, "t3", 0.0), (3, 1280, "outlier", 0.0),
    (4099, 256, "normal", 1e-5)])
def test_matches_oracle(dev, n, k, dist, eps):
    check(synth.fp_weights(n + k, n, k, dist), eps, dev)


def test_full_gate_up_tensor(dev):
    # 17920 x 1536: past every partial-sum workgroup's first share
    check(synth.fp_weights(7, 17920, 1536, "normal"), 1e-5, dev)


def test_all_zero_tensor(dev):
    for eps in (0.0, 1e-5):
        p, g = run(np.zeros((5, 256), np.float32), eps, dev)
        assert g == 0 and (p == 0x55).all()


def test_deterministic_and_workspace_contents_irrelevant(dev):
    w = synth.fp_weights(3, 600, 1536, "t3")
    a = run(w, 0.0, dev, poison=True)
    b = run(w, 0.0, dev, poison=False)
    assert a[1].view(np.uint32) == b[1].view(np.uint32)
    np.testing.assert_array_equal(a[0], b[0])


def test_ternarized_weights_feed_the_matmul(dev):
    # fp32 W -> bt_ternarize -> device repack -> GEMV and GEMM with the returned scale
    n, k = 2048, 1536
    w = synth.fp_weights(11, n, k, "normal")
    codes, gamma = oracle.ternarize_ref(w, 1e-5)
    packed, scale = bt.ternarize(torch.from_numpy(w).to(dev), 1e-5)
    wdev = bt.repack_ternary(packed, n, k)
    s = float(scale.cpu().numpy()[0])
    assert np.float32(s) == gamma
    for m in (1, 48):
        x = synth.small_problem(12, m, 16, k)["x"]
        ref = oracle.forward_ref(x, codes, gamma, "f64")
        q = bt.quantize_act(torch.from_numpy(x).to(dev))
        y, acc = bt.ternary_matmul(*q, wdev, n, s, want_acc=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
        yr = ref["y"]
        got = y.cpu().numpy()
        nz = yr != 0
        assert (got[~nz] == 0).all()
        assert (np.abs(got[nz] - yr[nz]) <= 1e-6 * np.abs(yr[nz])).all()


def test_grouped_plan_matches_single_calls_and_oracle(dev):
    """A grouped plan over tensors of every size class (the decoder's four
    shapes, ragged small ones, an all-zero one), one eps: each tensor's packed
    bytes and scale equal bt_ternarize's bit for bit, and the oracle's for a
    sample; relaunched after the outputs are poisoned, the same again."""
    shapes = [(2048, 1536, "normal"), (1536, 1536, "outlier"), (17920, 1536, "t3"),
              (1536, 8960, "normal"), (17, 128, "t3"), (1, 384, "normal"), (4099, 256, "outlier")]
    eps = 1e-5
    ws_ = [synth.fp_weights(40 + i, n, k, dist) for i, (n, k, dist) in enumerate(shapes)]
    ws_.append(np.zeros((5, 256), np.float32))
    items = []
    for w in ws_:
        n, k = w.shape
        items.append((torch.from_numpy(w).to(dev),
                      torch.empty(n * k // 4, dtype=torch.uint8, device=dev),
                      torch.empty(1, dtype=torch.float32, device=dev)))
    plan = bt.TernarizePlan(items, eps)
    for rep in range(2):
        for _, p, sc in items:
            p.fill_(0xFF)
            sc.fill_(float("nan"))
        plan.launch()
        torch.cuda.synchronize()
        for i, (w, p, sc) in enumerate(items):
            want_p, want_g = bt.ternarize(w, eps)
            torch.cuda.synchronize()
            assert torch.equal(p, want_p), (rep, i)
            assert sc.cpu().numpy().view(np.uint32)[0] == want_g.cpu().numpy().view(np.uint32)[0]
    for i in (0, len(items) - 1, len(items) - 2):
        w = ws_[i]
        want_p, want_g = oracle.ternarize_pack_ref(w, eps)
        got_p = items[i][1].cpu().numpy().reshape(want_p.shape)
        np.testing.assert_array_equal(got_p, want_p)
        assert np.float32(items[i][2].cpu().numpy()[0]) == want_g
