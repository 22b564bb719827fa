"""Long prefill, every output of every projection: 4096 tokens through all 28
layers x 4 projections of the decoder (qkv 1536->2048, o 1536->1536, gate_up
1536->17920, down 8960->1536), weights with P(-1, 0, +1) = (0.2, 0.6, 0.2),
activations Student-t with 3 degrees of freedom drawn on the GPU exactly as the
benchmark draws them.

The method's result is an exact integer sum followed by one fp32 rescale
("VibeVoice-ASR-BitNet Technical Report", section 2.4.2 and Figure 4: integer
multiply-add, horizontal sum; blog post "Paper 說支援 ARM…", fourth stage: an
optimized kernel must reproduce the plain element-wise product bit for bit).
So per projection: q, d and the row sums of the quantization, and the int32
accumulators, equal the oracle's in every element; y is within 1e-6 relative
(exactly 0 where the oracle's is 0).

Each projection runs in the launch configuration the benchmark times (one
quantize launch, then the GEMM the library picks for the shape: the persistent
kernel for gate_up, the tiled kernels for the others, no accumulator output).
A second GEMM launch that also writes the accumulators gives the int32 sums;
its y must equal the first launch's bit for bit. The same layer also runs as
one grouped quantization launch and one grouped GEMM launch, compared with the
oracle the same way. The oracle's exact fp64-BLAS product is itself checked
against int64 dot products on 1000 random (m, n) pairs, all of row 0 and all
of column 0.

One layer at a time is generated and run, and one projection at a time is
compared, so the host never holds more than one projection's oracle arrays.
A last test runs the whole stack in the benchmark's grouped form and compares
it with the per-projection launches on the GPU.
"""

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import ternary_weight_decoder_bt_amd as bt  # noqa: E402

M = 4096
RTOL = 1e-6
POISON_I32 = np.iinfo(np.int32).min


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _exact(name, got, want):
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches; first {i}: got {got[i]} "
                             f"want {want[i]}")


def _rel(name, got, want):
    assert np.isfinite(got).all(), f"{name}: non-finite output (unwritten element?)"
    zero = want == 0
    assert (got[zero] == 0).all(), f"{name}: nonzero where the oracle is exactly 0"
    g, w = got[~zero].astype(np.float64), want[~zero].astype(np.float64)
    rel = np.abs(g - w) / np.abs(w)
    assert rel.size == 0 or rel.max() <= RTOL, f"{name}: max rel err {rel.max():.3e}"


def _launch_layer(dev, layer):
    """The layer's four projections, each in the benchmark's per-projection launch
    configuration (quantize, GEMM without and with accumulators), and the same four
    as one grouped quantization launch and one grouped GEMM launch."""
    singles, gq, gm = [], [], []
    for proj in range(len(synth.PROJECTIONS)):
        name, k, n = synth.PROJECTIONS[proj]
        c = synth.long_prefill_problem(layer, proj, M, with_x=False)
        x_dev = synth.device_student_t3(M, k, synth.CFG_LONG, layer, proj, dev)
        wdev = bt.repack_ternary(torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev),
                                 n, k)
        r = {"name": name, "n": n, "k": k, "w": c["w"], "s": c["w_scale"], "x": x_dev,
             "wdev": wdev}
        r["xq"] = torch.full((M, k), 99, dtype=torch.int8, device=dev)
        r["xs"] = torch.full((M,), float("nan"), dtype=torch.float32, device=dev)
        r["xsum"] = torch.full((M,), POISON_I32, dtype=torch.int32, device=dev)
        bt.quantize_act(x_dev, r["xq"], r["xs"], r["xsum"])
        ws = bt.new_workspace(M, n, k, dev)
        r["y1"] = torch.full((M, n), float("nan"), dtype=torch.float32, device=dev)
        bt.ternary_matmul(r["xq"], r["xs"], r["xsum"], wdev, n, r["s"], y=r["y1"], workspace=ws)
        r["y2"] = torch.full((M, n), float("nan"), dtype=torch.float32, device=dev)
        r["acc"] = torch.full((M, n), POISON_I32, dtype=torch.int32, device=dev)
        bt.ternary_matmul(r["xq"], r["xs"], r["xsum"], wdev, n, r["s"], y=r["y2"], acc=r["acc"],
                          workspace=ws)
        g = {"xq": torch.full((M, k), 99, dtype=torch.int8, device=dev),
             "xscale": torch.full((M,), float("nan"), dtype=torch.float32, device=dev),
             "xsum": torch.full((M,), POISON_I32, dtype=torch.int32, device=dev),
             "y": torch.full((M, n), float("nan"), dtype=torch.float32, device=dev),
             "acc": torch.full((M, n), POISON_I32, dtype=torch.int32, device=dev),
             "wdev": wdev, "n": n, "w_scale": r["s"]}
        gq.append((x_dev, g["xq"], g["xscale"], g["xsum"]))
        gm.append(g)
        r["g"] = g
        singles.append(r)
    bt.QuantPlan(gq).launch()
    bt.MatmulPlan(gm).launch()
    torch.cuda.synchronize()
    return singles


def _check_projection(layer, r):
    tag = f"layer {layer} {r['name']} (M={M}, N={r['n']}, K={r['k']})"
    print(f"long prefill parity: {tag}", flush=True)
    w, s, g = r["w"], r["s"], r["g"]
    x = r["x"].cpu().numpy()
    q, d, qs = oracle.quantize_ref(x)
    del x
    for kind, xq, xs, xsum in (("", r["xq"], r["xs"], r["xsum"]),
                               (" grouped", g["xq"], g["xscale"], g["xsum"])):
        _exact(f"{tag}{kind} q", xq.cpu().numpy(), q)
        _exact(f"{tag}{kind} d", xs.cpu().numpy(), d)
        _exact(f"{tag}{kind} qsum", xsum.cpu().numpy(), qs)

    acc_ref = oracle.matmul_ref(q, w, "f64")
    # the oracle's exact-BLAS product against int64 dot products
    rng = np.random.default_rng(1000 * layer + r["n"] + r["k"])
    rows = rng.integers(0, M, 1000)
    cols = rng.integers(0, r["n"], 1000)
    _exact(f"{tag} oracle f64 vs brute", acc_ref[rows, cols],
           oracle.matmul_rows_cols(q, w, rows, cols))
    _exact(f"{tag} oracle row 0", acc_ref[:1], oracle.matmul_ref(q[:1], w, "int64"))
    _exact(f"{tag} oracle column 0", acc_ref[:, :1], oracle.matmul_ref(q, w[:1], "int64"))

    _exact(f"{tag} acc", r["acc"].cpu().numpy(), acc_ref)
    _exact(f"{tag} grouped acc", g["acc"].cpu().numpy(), acc_ref)
    y_ref = oracle.dequant_ref(acc_ref, d, s)
    del acc_ref
    y1 = r["y1"].cpu().numpy()
    _rel(f"{tag} y", y1, y_ref)
    _rel(f"{tag} grouped y", g["y"].cpu().numpy(), y_ref)
    _exact(f"{tag} y with and without acc", r["y2"].cpu().numpy(), y1)


@pytest.mark.parametrize("layer", range(synth.N_LAYERS))
def test_long_prefill_layer_every_output(dev, layer):
    """Per-projection launches and the layer's grouped launches, every output
    against the oracle."""
    for r in _launch_layer(dev, layer):
        _check_projection(layer, r)
    torch.cuda.empty_cache()


def test_long_prefill_stack_grouped_matches_per_projection(dev):
    """The whole stack as the benchmark's grouped form (one quantization plan over
    the 112 inputs, one GEMM plan over the 112 projections) equals the
    per-projection launches, which the tests above compare with the oracle, in
    every output bit for bit (compared on the GPU)."""
    per, gq, gm = [], [], []
    for layer in range(synth.N_LAYERS):
        for proj in range(len(synth.PROJECTIONS)):
            _, k, n = synth.PROJECTIONS[proj]
            c = synth.long_prefill_problem(layer, proj, M, with_weights=False, with_x=False)
            w = synth.long_prefill_problem(layer, proj, M, with_x=False)["w"]
            x = synth.device_student_t3(M, k, synth.CFG_LONG, layer, proj, dev)
            wdev = bt.repack_ternary(torch.from_numpy(bt.pack_ternary(w).reshape(-1)).to(dev),
                                     n, k)
            xq, xs, xsum = bt.quantize_act(x)
            y = bt.ternary_matmul(xq, xs, xsum, wdev, n, c["w_scale"],
                                  workspace=bt.new_workspace(M, n, k, dev))
            g = {"xq": torch.full((M, k), 99, dtype=torch.int8, device=dev),
                 "xscale": torch.full((M,), float("nan"), dtype=torch.float32, device=dev),
                 "xsum": torch.full((M,), POISON_I32, dtype=torch.int32, device=dev),
                 "y": torch.full((M, n), float("nan"), dtype=torch.float32, device=dev),
                 "wdev": wdev, "n": n, "w_scale": c["w_scale"]}
            gq.append((x, g["xq"], g["xscale"], g["xsum"]))
            gm.append(g)
            per.append((xq, xs, xsum, y))
    print("long prefill grouped stack: 112 projections launched one by one", flush=True)
    bt.QuantPlan(gq).launch()
    bt.MatmulPlan(gm).launch()
    torch.cuda.synchronize()
    print("long prefill grouped stack: grouped launches done", flush=True)
    for i, ((xq, xs, xsum, y), g) in enumerate(zip(per, gm)):
        assert torch.equal(g["xq"], xq), i
        assert torch.equal(g["xscale"], xs), i
        assert torch.equal(g["xsum"], xsum), i
        assert torch.equal(g["y"], y), i
    del per, gq, gm
    torch.cuda.empty_cache()
