"""The C ABI from a plain C program (no Python, no torch on the calling side).

`tests/c/bt_c_abi_run.c`, built by `__graft_entry__.build()` with gcc against
`include/bt.h` and `libbt.so`, packs on the host, repacks, quantizes and
multiplies with hipMalloc'd buffers on its own stream, runs the fused call
where M <= 16, and writes every output to a file. Here those outputs are
compared with the CPU oracle, to the same bar as the other parity tests: q,
d, row sums and accumulators bit-exact, y within 1e-6 relative (exactly 0
where the oracle is 0).
"""

import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNNER = os.path.join(ROOT, "tests", "c", "bt_c_abi_run")
RTOL = 1e-6


def _gpu_present():
    torch = pytest.importorskip("torch")
    return torch.cuda.device_count() > 0


def _run(x, w, w_scale):
    m, k = x.shape
    n = w.shape[0]
    with tempfile.TemporaryDirectory() as d:
        src, dst = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(src, "wb") as f:
            f.write(np.array([m, n, k], dtype="<i8").tobytes())
            f.write(np.array([w_scale], dtype="<f4").tobytes())
            f.write(np.ascontiguousarray(x, dtype="<f4").tobytes())
            f.write(np.ascontiguousarray(w, dtype=np.int8).tobytes())
        res = subprocess.run([RUNNER, src, dst], capture_output=True, text=True, timeout=120)
        assert res.returncode == 0, res.stderr
        raw = open(dst, "rb").read()
    off = 0

    def take(dtype, count):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=off)
        off += a.nbytes
        return a

    out = {"status": take("<i4", 5)}
    for prefix in ("", "fused_"):
        out[prefix + "q"] = take(np.int8, m * k).reshape(m, k)
        out[prefix + "d"] = take("<f4", m)
        out[prefix + "qsum"] = take("<i4", m)
        out[prefix + "acc"] = take("<i4", m * n).reshape(m, n)
        out[prefix + "y"] = take("<f4", m * n).reshape(m, n)
    assert off == len(raw)
    return out


def _assert_rel(name, got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert np.isfinite(got).all(), name
    zero = want == 0
    assert (got[zero] == 0).all(), f"{name}: nonzero where the oracle is exactly 0"
    rel = np.abs(got[~zero] - want[~zero]) / np.abs(want[~zero])
    assert rel.size == 0 or rel.max() <= RTOL, f"{name}: max rel err {rel.max():.3e}"


@pytest.mark.parametrize("m,n,k,seed", [
    (3, 100, 384, 1),      # GEMV, ragged N
    (16, 40, 8960, 2),     # GEMV whose activations split K over workgroups (workspace)
    (130, 300, 640, 3),    # GEMM, ragged tiles
])
def test_c_caller_matches_oracle(m, n, k, seed):
    if not _gpu_present():
        pytest.skip("no GPU")
    assert os.path.exists(RUNNER), f"{RUNNER} is not built; run __graft_entry__.build()"
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    w_scale = 0.02
    out = _run(x, w, w_scale)
    assert out["status"].tolist() == [0, 0, 0, 0, 0]
    ref = oracle.forward_ref(x, w, w_scale, "int64")
    prefixes = ("", "fused_") if m <= 16 else ("",)
    for p in prefixes:
        np.testing.assert_array_equal(out[p + "q"], ref["q"], err_msg=p + "q")
        np.testing.assert_array_equal(out[p + "d"], ref["d"], err_msg=p + "d")
        np.testing.assert_array_equal(out[p + "qsum"], ref["qsum"], err_msg=p + "qsum")
        np.testing.assert_array_equal(out[p + "acc"], ref["acc"], err_msg=p + "acc")
        _assert_rel(p + "y", out[p + "y"], ref["y"])
