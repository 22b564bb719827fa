"""Every launch goes to the stream it is given. The whole path (repack,
quantize, GEMV and GEMM with a K split and its reduce launch, the grouped plan
with its atomics, the I8_S product) runs on a side stream while
the current stream is left alone; only that side stream is synchronized before
the results are read, and they must be the oracle's. A launch on another stream
would race with the side stream's producers (the inputs are written on the side
stream just before)."""

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


@pytest.mark.parametrize("m,n,k", [(16, 1536, 8960), (150, 1536, 8960), (4096, 2048, 1536)])
def test_matmul_on_side_stream(dev, m, n, k):
    c = synth.small_problem(90, m, n, k, "t3")
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    packed_h = torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1))
    x_h = torch.from_numpy(c["x"])
    s = torch.cuda.Stream()
    need = bt.matmul_workspace_bytes(m, n, k)
    with torch.cuda.stream(s):
        # inputs produced on the side stream itself, just before their use
        packed = packed_h.to(dev, non_blocking=False)
        x = x_h.to(dev, non_blocking=False)
        ws = torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device=dev)
        y = torch.full((m, n), float("nan"), device=dev)
        acc = torch.full((m, n), -1, dtype=torch.int32, device=dev)
    wdev = bt.repack_ternary(packed, n, k, stream=s)
    xq, xs, xsum = bt.quantize_act(x, stream=s)
    bt.ternary_matmul(xq, xs, xsum, wdev, n, c["w_scale"], y=y, acc=acc,
                      workspace=ws if need else None, stream=s)
    s.synchronize()
    assert np.array_equal(xq.cpu().numpy(), ref["q"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert np.array_equal(y.cpu().numpy(), ref["y"])


def test_grouped_plan_and_i8s_on_side_stream(dev):
    cases = [synth.decode_problem(0, proj, 16) for proj in range(4)]
    s = torch.cuda.Stream()
    items, refs = [], []
    with torch.cuda.stream(s):
        for c in cases:
            n, k = c["N"], c["K"]
            wdev = bt.repack_ternary(torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev),
                                     n, k, stream=s)
            items.append({"x": torch.from_numpy(c["x"]).to(dev), "wdev": wdev, "n": n,
                          "w_scale": c["w_scale"],
                          "y": torch.full((16, n), float("nan"), device=dev)})
            refs.append(oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64"))
        plan = bt.MatmulPlan(items)
    for _ in range(3):
        plan.launch(stream=s)
    # the I8_S product on the same stream
    rng = np.random.default_rng(91)
    x8 = synth.small_problem(91, 300, 16, 256, "t3")["x"]
    w8 = rng.integers(-128, 128, (200, 256), dtype=np.int8)
    with torch.cuda.stream(s):
        xq, xs_, _ = bt.quantize_act(torch.from_numpy(x8).to(dev), stream=s)
        w8dev = bt.repack_int8(torch.from_numpy(w8).to(dev), stream=s)
        y8 = bt.int8_matmul(xq, xs_, w8dev, 200, 0.01, stream=s)
    s.synchronize()
    for it, ref in zip(items, refs):
        got = it["y"].cpu().numpy()
        nz = ref["y"] != 0
        assert (got[~nz] == 0).all()
        assert (np.abs(got[nz] - ref["y"][nz]) <= 1e-6 * np.abs(ref["y"][nz])).all()
    assert np.array_equal(y8.cpu().numpy(), oracle.i8s_forward_ref(x8, w8, np.float32(0.01))["y"])
