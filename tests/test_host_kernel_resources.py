"""Every kernel of libbt compiles for gfx950 without private (scratch) memory.

The kernels' pipelines wait on the vector-memory counter with static counts
(loads, LDS copies and stores complete in issue order), and the persistent
GEMM sits at the full 256-register budget of two waves per SIMD. A spilled
register is stored to and reloaded from scratch through that same in-order
queue, and the wait for a reload drains every load in flight: a small edit
that makes the compiler spill slows a kernel down without changing a single
output. This host-only check compiles each HIP source of the library with the
build's own flags and reads the compiler's per-kernel resource report.
"""

import os
import re
import subprocess
import tempfile

import pytest

from ternary_weight_decoder_bt_amd import _build

FUNC = re.compile(r"remark: Function Name: (\S+)")
FIELD = re.compile(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|VGPRs Spill|Occupancy \[waves/SIMD\]): (\d+)")


def _resources(source: str, workdir: str) -> dict:
    flags = [f for f in _build.FLAGS if f != "-shared"]
    cmd = [_build.hipcc(), *flags, "-I", _build.INCLUDE, "-I", _build.CSRC, "-c",
           os.path.join(_build.CSRC, source), "-o", os.path.join(workdir, source + ".o"),
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = FUNC.search(line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = FIELD.search(line)
        if m and cur is not None:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def resources():
    try:
        _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available")
    sources = [s for s in _build.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as d:
        return {s: _resources(s, d) for s in sources}


def test_every_kernel_is_free_of_scratch(resources):
    seen = 0
    for source, kernels in resources.items():
        assert kernels, f"no kernel resource report for {source}"
        for name, r in kernels.items():
            seen += 1
            assert r.get("ScratchSize [bytes/lane]", -1) == 0, (source, name, r)
            assert r.get("VGPRs Spill", -1) == 0, (source, name, r)
    assert seen >= 20


def test_occupancy_of_the_hot_kernels(resources):
    """The persistent GEMM runs two workgroups of four waves per compute unit
    (two waves per SIMD), the decode GEMV at least four waves per SIMD."""
    gemm = resources["bt_gemm.hip"]
    persistent = [n for n in gemm if "gemm_persistent" in n]
    assert len(persistent) == 2
    for n in persistent:
        assert gemm[n]["Occupancy [waves/SIMD]"] >= 2, (n, gemm[n])
    kern = resources["bt_kernels.hip"]
    grouped = [n for n in kern if "gemv_grouped_kernel" in n]
    assert len(grouped) == 2
    for n in grouped:
        assert kern[n]["Occupancy [waves/SIMD]"] >= 4, (n, kern[n])
