"""Build libbt.so (the matmul path) and libbt_ceilings.so (hardware ceiling
measurements) in-tree with hipcc for gfx950 (MI355X)."""

from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libbt.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ("bt_host.cpp", "bt_kernels.hip", "bt_gemm.hip", "bt_ternarize.hip")
CEILINGS_LIB_PATH = os.path.join(PKG_DIR, "libbt_ceilings.so")
CEILINGS_SOURCES = ("bt_ceilings.hip",)

# -ffp-contract=off: the quantizer's rounding decision must see the rounded
#   fp32 product x * (127 / a), never a fused multiply-add of it.
# -packed-fp32-ops off: no packed fp32 instructions in any kernel.
# fp32 denormals are kept (no flush flag), and division stays correctly rounded.
FLAGS = (
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile libbt.so and libbt_ceilings.so next to this file; returns the
    path of libbt.so."""
    _compile(SOURCES, LIB_PATH, verbose)
    _compile(CEILINGS_SOURCES, CEILINGS_LIB_PATH, verbose)
    return LIB_PATH


def _compile(sources, lib_path: str, verbose: bool) -> None:
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        print(" ".join(cmd))
        print(res.stdout)
        # the host pass does not know the packed-fp32 feature; that warning is harmless
        print("\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, lib_path)


if __name__ == "__main__":
    print(build(verbose=True))
