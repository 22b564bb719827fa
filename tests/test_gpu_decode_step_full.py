"""The whole decode step at full size, every output: the 112 projections of the
28-layer decoder at M=1 (qkv 1536->2048, o 1536->1536, gate_up 1536->17920,
down 8960->1536; weights uniform ternary, scales ~U(0.01, 0.05), activations
N(0,1) with 0.1% x20), exactly the benchmark's inputs, in each of the four
forms the benchmark times:

- one grouped launch with the quantization fused (the headline),
- a grouped quantization launch then a grouped GEMV launch,
- the dependent chain of 112 fused single calls,
- the dependent chain of 112 (quantize, GEMV) single-call pairs.

Bar ("VibeVoice-ASR-BitNet Technical Report", section 2.4.2 and Figure 4: an
exact integer sum, then one fp32 rescale): q, d, row sums and the int32
accumulators equal the oracle's in every element, y within 1e-6 relative
(exactly 0 where the oracle's is 0). Outputs are poisoned before every form.
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
def step():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    probs = []
    for layer in range(synth.N_LAYERS):
        for proj in range(len(synth.PROJECTIONS)):
            c = synth.decode_problem(layer, proj)
            m, k, n = c["M"], c["K"], c["N"]
            ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "int64")
            packed = torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev)
            p = {"tag": f"layer {layer} {c['name']}", "m": m, "k": k, "n": n,
                 "s": c["w_scale"], "ref": ref, "x": torch.from_numpy(c["x"]).to(dev),
                 "wdev": bt.repack_ternary(packed, n, k),
                 "xq": torch.empty((m, k), dtype=torch.int8, device=dev),
                 "xs": torch.empty(m, dtype=torch.float32, device=dev),
                 "xsum": torch.empty(m, dtype=torch.int32, device=dev),
                 "y": torch.empty((m, n), dtype=torch.float32, device=dev),
                 "acc": torch.empty((m, n), dtype=torch.int32, device=dev)}
            probs.append(p)
    torch.cuda.synchronize()
    return probs


def _poison(probs):
    for p in probs:
        p["xq"].fill_(99)
        p["xs"].fill_(float("nan"))
        p["xsum"].fill_(POISON_I32)
        p["y"].fill_(float("nan"))
        p["acc"].fill_(POISON_I32)


def _check(probs, form):
    torch.cuda.synchronize()
    for p in probs:
        ref, tag = p["ref"], f"{form}: {p['tag']}"
        for name, got, want in (("q", p["xq"], ref["q"]), ("d", p["xs"], ref["d"]),
                                ("qsum", p["xsum"], ref["qsum"]), ("acc", p["acc"], ref["acc"])):
            g = got.cpu().numpy()
            assert np.array_equal(g, want), f"{tag} {name}: {int((g != want).sum())} mismatches"
        y = p["y"].cpu().numpy().astype(np.float64)
        want = ref["y"].astype(np.float64)
        zero = want == 0
        assert np.isfinite(y).all(), tag
        assert (y[zero] == 0).all(), tag
        rel = np.abs(y[~zero] - want[~zero]) / np.abs(want[~zero])
        assert rel.size == 0 or rel.max() <= RTOL, f"{tag} y: max rel err {rel.max():.3e}"


def _items(probs, fused):
    out = []
    for p in probs:
        it = {"xq": p["xq"], "xscale": p["xs"], "xsum": p["xsum"], "wdev": p["wdev"], "n": p["n"],
              "w_scale": p["s"], "y": p["y"], "acc": p["acc"]}
        if fused:
            it["x"] = p["x"]
        out.append(it)
    return out


def test_decode_step_grouped_fused(step):
    plan = bt.MatmulPlan(_items(step, True))
    _poison(step)
    plan.launch()
    _check(step, "grouped fused")


def test_decode_step_grouped_two_launch(step):
    qplan = bt.QuantPlan([(p["x"], p["xq"], p["xs"], p["xsum"]) for p in step])
    plan = bt.MatmulPlan(_items(step, False))
    _poison(step)
    qplan.launch()
    plan.launch()
    _check(step, "grouped two-launch")


def test_decode_step_chain_fused(step):
    _poison(step)
    for p in step:
        bt.ternary_matmul_fused(p["x"], p["wdev"], p["n"], p["s"], y=p["y"], acc=p["acc"],
                                xq=p["xq"], xscale=p["xs"], xsum=p["xsum"])
    _check(step, "chain fused")


def test_decode_step_chain_two_launch(step):
    _poison(step)
    for p in step:
        bt.quantize_act(p["x"], p["xq"], p["xs"], p["xsum"])
        bt.ternary_matmul(p["xq"], p["xs"], p["xsum"], p["wdev"], p["n"], p["s"], y=p["y"],
                          acc=p["acc"])
    _check(step, "chain two-launch")
