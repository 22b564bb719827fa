"""The library's launches inside a captured HIP graph: every replay must give
exactly the eager results (the kernels take the caller's stream and issue no
memset, allocation or host synchronization, so they are capturable).

Each replay is preceded by eager work on the same buffers (outputs poisoned
with NaN, an eager launch into other buffers) and a synchronization. The last
replays follow new activations written into the captured input buffers.
"""

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import ternary_weight_decoder_bt_amd as bt  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _weights(c, dev):
    n, k = c["w"].shape
    packed = torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev)
    return bt.repack_ternary(packed, n, k)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replays_match_eager(dev):
    # a grouped decode step (fused and two-launch), a split-K GEMV and a GEMM
    cases = [synth.decode_problem(0, proj) for proj in range(4)]
    ws = [_weights(c, dev) for c in cases]
    xs = [torch.from_numpy(c["x"]).to(dev) for c in cases]

    def outs(c):
        m, k, n = c["M"], c["K"], c["N"]
        return {"xq": torch.empty((m, k), dtype=torch.int8, device=dev),
                "xscale": torch.empty(m, dtype=torch.float32, device=dev),
                "xsum": torch.empty(m, dtype=torch.int32, device=dev),
                "y": torch.empty((m, n), dtype=torch.float32, device=dev),
                "acc": torch.empty((m, n), dtype=torch.int32, device=dev)}

    two = [outs(c) for c in cases]
    fused = [outs(c) for c in cases]
    qplan = bt.QuantPlan([(x, o["xq"], o["xscale"], o["xsum"]) for x, o in zip(xs, two)])
    mplan = bt.MatmulPlan([dict(o, wdev=w, n=c["N"], w_scale=c["w_scale"])
                           for o, w, c in zip(two, ws, cases)])
    fplan = bt.MatmulPlan([dict(o, wdev=w, n=c["N"], w_scale=c["w_scale"], x=x)
                           for o, w, c, x in zip(fused, ws, cases, xs)])
    sk = synth.small_problem(21, 16, 1536, 8960)
    sk_w, sk_x = _weights(sk, dev), torch.from_numpy(sk["x"]).to(dev)
    sk_q = bt.quantize_act(sk_x)
    sk_ws = bt.new_workspace(16, 1536, 8960, dev)
    assert sk_ws is not None                      # 16 rows x 8960: K is split
    sk_y = torch.empty((16, 1536), dtype=torch.float32, device=dev)
    gm = synth.small_problem(22, 200, 2048, 1536, "t3")
    gm_w, gm_x = _weights(gm, dev), torch.from_numpy(gm["x"]).to(dev)
    gm_q = [torch.empty((200, 1536), dtype=torch.int8, device=dev),
            torch.empty(200, dtype=torch.float32, device=dev),
            torch.empty(200, dtype=torch.int32, device=dev)]
    gm_y = torch.empty((200, 2048), dtype=torch.float32, device=dev)

    def work():
        qplan.launch()
        mplan.launch()
        fplan.launch()
        bt.ternary_matmul(*sk_q, sk_w, 1536, sk["w_scale"], y=sk_y, workspace=sk_ws)
        bt.quantize_act(gm_x, *gm_q)
        bt.ternary_matmul(*gm_q, gm_w, 2048, gm["w_scale"], y=gm_y)

    def snapshot():
        torch.cuda.synchronize()
        tensors = [t for o in two + fused for t in o.values()] + [sk_y, gm_y] + gm_q
        return [t.clone() for t in tensors]

    def poison():
        for o in two + fused:
            o["y"].fill_(float("nan"))
            o["acc"].fill_(-1)
            o["xq"].fill_(99)
        sk_y.fill_(float("nan"))
        sk_ws.fill_(0x5A)                         # partial slices are overwritten
        gm_y.fill_(float("nan"))
        gm_q[0].fill_(99)

    work()
    eager = snapshot()
    g = _capture(work)
    for rep in range(4):
        poison()
        # unrelated eager launch between replays
        bt.ternary_matmul(*sk_q, sk_w, 1536, sk["w_scale"], workspace=sk_ws)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for i, (a, b) in enumerate(zip(got, eager)):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                               b.view(torch.uint8) if b.dtype == torch.float32 else b), (rep, i)

    # New activations written into the captured input buffers: a replay must
    # follow them, as a decoder's step-by-step replays do. The eager launches
    # on the same new inputs give the expected bytes.
    def same(a, b):
        return torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                           b.view(torch.uint8) if b.dtype == torch.float32 else b)

    rng = np.random.default_rng(23)
    for rep in range(2):
        for x in xs + [gm_x]:
            x.copy_(torch.from_numpy(rng.standard_normal(tuple(x.shape)).astype(np.float32)))
        work()
        want = snapshot()
        poison()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for i, (a, b) in enumerate(zip(got, want)):
            assert same(a, b), ("new inputs", rep, i)
        # the decode outputs did change with the inputs
        assert not same(want[3], eager[3]) and not same(want[-4], eager[-4])


def test_graph_grouped_prefill_and_noalloc(dev):
    """A grouped prefill (grouped quantization, grouped GEMM plan over ragged
    projections with different K, one of them split into K ranges whose reduce
    launch is part of the plan's launch) and the allocation-free matmul on a
    split shape, captured once: every replay, after eager work and a poisoning
    of the outputs, equals the eager launches byte for byte."""
    shapes = [(600, 2048, 1536), (300, 1536, 8960), (129, 130, 384)]
    cases = [synth.small_problem(30 + i, m, n, k, "t3") for i, (m, n, k) in enumerate(shapes)]
    ws = [_weights(c, dev) for c in cases]
    xs = [torch.from_numpy(c["x"]).to(dev) for c in cases]
    outs = [{"xq": torch.empty(c["x"].shape, dtype=torch.int8, device=dev),
             "xscale": torch.empty(c["x"].shape[0], dtype=torch.float32, device=dev),
             "xsum": torch.empty(c["x"].shape[0], dtype=torch.int32, device=dev),
             "y": torch.empty((c["x"].shape[0], c["N"]), dtype=torch.float32, device=dev)}
            for c in cases]
    qplan = bt.QuantPlan([(x, o["xq"], o["xscale"], o["xsum"]) for x, o in zip(xs, outs)])
    gplan = bt.MatmulPlan([dict(o, wdev=w, n=c["N"], w_scale=c["w_scale"])
                           for o, w, c in zip(outs, ws, cases)])
    na = synth.small_problem(35, 16, 1536, 8960)
    assert bt.matmul_workspace_bytes(16, 1536, 8960) > 0      # K is split
    na_w, na_q = _weights(na, dev), bt.quantize_act(torch.from_numpy(na["x"]).to(dev))
    na_y = torch.empty((16, 1536), dtype=torch.float32, device=dev)

    def work():
        qplan.launch()
        gplan.launch()
        bt.ternary_matmul_noalloc(*na_q, na_w, 1536, na["w_scale"], na_y)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for o in outs for t in o.values()] + [na_y.clone()]

    work()
    eager = snapshot()
    g = _capture(work)
    for rep in range(3):
        for o in outs:
            o["y"].fill_(float("nan"))
            o["xq"].fill_(99)
        na_y.fill_(float("nan"))
        bt.ternary_matmul(*na_q, na_w, 1536, na["w_scale"],
                          workspace=bt.new_workspace(16, 1536, 8960, dev))
        torch.cuda.synchronize()
        g.replay()
        for i, (a, b) in enumerate(zip(snapshot(), eager)):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                               b.view(torch.uint8) if b.dtype == torch.float32 else b), (rep, i)
