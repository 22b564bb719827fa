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
its y must equal the first launch's bit for bit. The oracle's exact fp64-BLAS
product is itself checked against int64 dot products on 1000 random (m, n)
pairs, all of row 0 and all of column 0.

One projection at a time is generated, run and compared, so the host never
holds more than one projection's tensors.
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


def _projection(dev, layer, proj):
    name, k, n = synth.PROJECTIONS[proj]
    tag = f"layer {layer} {name} (M={M}, N={n}, K={k})"
    print(f"long prefill parity: {tag}", flush=True)
    c = synth.long_prefill_problem(layer, proj, M, with_x=False)
    w, s = c["w"], c["w_scale"]
    x_dev = synth.device_student_t3(M, k, synth.CFG_LONG, layer, proj, dev)
    wdev = bt.repack_ternary(torch.from_numpy(bt.pack_ternary(w).reshape(-1)).to(dev), n, k)

    xq = torch.full((M, k), 99, dtype=torch.int8, device=dev)
    xs = torch.full((M,), float("nan"), dtype=torch.float32, device=dev)
    xsum = torch.full((M,), POISON_I32, dtype=torch.int32, device=dev)
    bt.quantize_act(x_dev, xq, xs, xsum)
    ws = bt.new_workspace(M, n, k, dev)
    y1 = torch.full((M, n), float("nan"), dtype=torch.float32, device=dev)
    bt.ternary_matmul(xq, xs, xsum, wdev, n, s, y=y1, workspace=ws)
    y2 = torch.full((M, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((M, n), POISON_I32, dtype=torch.int32, device=dev)
    bt.ternary_matmul(xq, xs, xsum, wdev, n, s, y=y2, acc=acc, workspace=ws)
    torch.cuda.synchronize()
    x = x_dev.cpu().numpy()
    del x_dev, wdev, ws

    q, d, qs = oracle.quantize_ref(x)
    _exact(f"{tag} q", xq.cpu().numpy(), q)
    _exact(f"{tag} d", xs.cpu().numpy(), d)
    _exact(f"{tag} qsum", xsum.cpu().numpy(), qs)
    del xq, xs, xsum, x

    acc_ref = oracle.matmul_ref(q, w, "f64")
    # the oracle's exact-BLAS product against int64 dot products
    rng = np.random.default_rng(1000 * layer + proj)
    rows = rng.integers(0, M, 1000)
    cols = rng.integers(0, n, 1000)
    _exact(f"{tag} oracle f64 vs brute", acc_ref[rows, cols],
           oracle.matmul_rows_cols(q, w, rows, cols))
    _exact(f"{tag} oracle row 0", acc_ref[:1], oracle.matmul_ref(q[:1], w, "int64"))
    _exact(f"{tag} oracle column 0", acc_ref[:, :1], oracle.matmul_ref(q, w[:1], "int64"))

    _exact(f"{tag} acc", acc.cpu().numpy(), acc_ref)
    y_ref = oracle.dequant_ref(acc_ref, d, s)
    del acc, acc_ref
    y1 = y1.cpu().numpy()
    _rel(f"{tag} y", y1, y_ref)
    _exact(f"{tag} y with and without acc", y2.cpu().numpy(), y1)


@pytest.mark.parametrize("layer", range(synth.N_LAYERS))
def test_long_prefill_layer_every_output(dev, layer):
    for proj in range(len(synth.PROJECTIONS)):
        _projection(dev, layer, proj)
    torch.cuda.empty_cache()
