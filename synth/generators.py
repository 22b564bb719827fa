"""Seeded synthetic workloads for the ternary-weight decoder matmul.

The technical report ("VibeVoice-ASR-BitNet Technical Report", sections 2.1
and 2.3.2) swaps the decoder for a 1.5B, 28-layer transformer (Qwen2.5-1.5B:
hidden size 1536, fused QKV 1536->2048, O 1536->1536, fused gate+up
1536->17920, down 8960->1536). The measured workloads of the pages (ASR
evaluation sets and 20-s clips, section 3.1) and the trained checkpoint are
not available, so every input here is synthetic with those shapes.

Every stream is drawn from ``PCG64(SeedSequence([cfg, layer, proj, stream]))``
so that one projection can be regenerated alone, on any host, byte for byte.
The single-GEMV workload uses ``default_rng(0)`` for activations and
``default_rng(1)`` for weights.

Nothing here packs, quantizes or multiplies: the weights come out as int8
values in {-1, 0, +1} (N rows of K, K contiguous), or as fp32 before
ternarization, and the activations as fp32 (M rows of K).
"""

from __future__ import annotations

import numpy as np

HIDDEN = 1536
N_LAYERS = 28
# (name, K = input features, N = output features) of one decoder layer.
PROJECTIONS = (
    ("qkv", 1536, 2048),
    ("o", 1536, 1536),
    ("gate_up", 1536, 17920),
    ("down", 8960, 1536),
)

STREAM_W, STREAM_X, STREAM_SCALE, STREAM_OUTLIER = 0, 1, 2, 3

# Workload ids (the first SeedSequence word).
CFG_SINGLE, CFG_DECODE, CFG_REMAINDER, CFG_PREFILL, CFG_LONG, CFG_FPW = 0, 1, 2, 3, 4, 5

REMAINDER_MS = (1, 2, 3, 4, 5, 7, 8, 16)


def projection_rng(cfg: int, layer: int, proj: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, layer, proj, stream])))


def ternary_weights(rng: np.random.Generator, n: int, k: int, p=None) -> np.ndarray:
    """int8 (n, k) with values in {-1, 0, +1}.

    ``p`` = (P(-1), P(0), P(+1)); None means uniform over the three values.
    """
    if p is None:
        return rng.integers(-1, 2, size=(n, k), dtype=np.int8)
    u = rng.random((n, k), dtype=np.float32)
    w = np.zeros((n, k), dtype=np.int8)
    w[u < np.float32(p[0])] = -1
    w[u >= np.float32(p[0] + p[1])] = 1
    return w


def _scale(cfg: int, layer: int, proj: int) -> np.float32:
    return np.float32(projection_rng(cfg, layer, proj, STREAM_SCALE).uniform(0.01, 0.05))


def _normal_with_outliers(cfg: int, layer: int, proj: int, m: int, k: int) -> np.ndarray:
    x = projection_rng(cfg, layer, proj, STREAM_X).standard_normal((m, k), dtype=np.float32)
    mask = projection_rng(cfg, layer, proj, STREAM_OUTLIER).random((m, k)) < 0.001
    x[mask] *= np.float32(20.0)
    return x


def config0() -> dict:
    """One GEMV: M=1, K=N=1536, x ~ N(0,1) (seed 0), W uniform ternary (seed 1), scale 0.02."""
    x = np.random.default_rng(0).standard_normal((1, HIDDEN), dtype=np.float32)
    w = np.random.default_rng(1).integers(-1, 2, size=(HIDDEN, HIDDEN), dtype=np.int8)
    return {"x": x, "w": w, "w_scale": np.float32(0.02), "M": 1, "K": HIDDEN, "N": HIDDEN}


def decode_problem(layer: int, proj: int, m: int = 1, *, with_weights: bool = True,
                   with_x: bool = True, cfg: int = CFG_DECODE) -> dict:
    """Decode-step projection: W uniform ternary, scale ~U(0.01,0.05), x ~ N(0,1) with 0.1% x20."""
    name, k, n = PROJECTIONS[proj]
    out = {"name": name, "M": m, "K": k, "N": n, "w_scale": _scale(cfg, layer, proj)}
    if with_weights:
        out["w"] = ternary_weights(projection_rng(cfg, layer, proj, STREAM_W), n, k)
    if with_x:
        out["x"] = _normal_with_outliers(cfg, layer, proj, m, k)
    return out


def decode_remainder_problem(proj_name: str, m: int) -> dict:
    """gate+up or down at a small batch M, distributed as the decode step (layer 0)."""
    proj = [p[0] for p in PROJECTIONS].index(proj_name)
    return decode_problem(0, proj, m, cfg=CFG_REMAINDER)


def prefill_problem(proj: int, m: int = 512, *, with_weights: bool = True,
                    with_x: bool = True) -> dict:
    """One-layer prefill: W with P(-1,0,+1) = (0.3,0.4,0.3), x ~ N(0,1)."""
    name, k, n = PROJECTIONS[proj]
    out = {"name": name, "M": m, "K": k, "N": n, "w_scale": _scale(CFG_PREFILL, 0, proj)}
    if with_weights:
        out["w"] = ternary_weights(projection_rng(CFG_PREFILL, 0, proj, STREAM_W), n, k,
                                   (0.3, 0.4, 0.3))
    if with_x:
        out["x"] = projection_rng(CFG_PREFILL, 0, proj, STREAM_X).standard_normal(
            (m, k), dtype=np.float32)
    return out


def long_prefill_problem(layer: int, proj: int, m: int = 4096, *, with_weights: bool = True,
                         with_x: bool = True) -> dict:
    """Long prefill: W with P = (0.2,0.6,0.2), x iid Student-t with 3 degrees of freedom."""
    name, k, n = PROJECTIONS[proj]
    out = {"name": name, "M": m, "K": k, "N": n, "w_scale": _scale(CFG_LONG, layer, proj)}
    if with_weights:
        out["w"] = ternary_weights(projection_rng(CFG_LONG, layer, proj, STREAM_W), n, k,
                                   (0.2, 0.6, 0.2))
    if with_x:
        out["x"] = projection_rng(CFG_LONG, layer, proj, STREAM_X).standard_t(
            3, size=(m, k)).astype(np.float32)
    return out


def device_student_t3(m: int, k: int, cfg: int, layer: int, proj: int, device):
    """x ~ Student-t with 3 degrees of freedom, drawn on the GPU with torch.

    t = z / sqrt(chi2_3 / 3) with chi2_3 the sum of three squared standard
    normals. Used where drawing gigabytes of activations on the host would
    dominate a benchmark's set-up time; the same seed always gives the same
    tensor on the same device and torch version.
    """
    import torch
    seed = int(np.random.SeedSequence([cfg, layer, proj, STREAM_X]).generate_state(1, np.uint64)[0]
               & np.uint64(2 ** 63 - 1))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn((m, k), generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros((m, k), device=device, dtype=torch.float32)
    for _ in range(3):
        chi += torch.randn((m, k), generator=g, device=device, dtype=torch.float32).square()
    return z / torch.sqrt(chi / 3)


def fp_weights(seed: int, n: int, k: int, dist: str = "normal") -> np.ndarray:
    """fp32 (n, k) full-precision weights before ternarization: N(0, s^2) with a
    seeded s ~ U(0.01, 0.05) ("normal"), the same with 0.1% of entries x10
    ("outlier"), or s * Student-t with 3 degrees of freedom ("t3")."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([CFG_FPW, seed, n, k])))
    s = np.float32(rng.uniform(0.01, 0.05))
    if dist == "normal":
        w = rng.standard_normal((n, k), dtype=np.float32)
    elif dist == "outlier":
        w = rng.standard_normal((n, k), dtype=np.float32)
        w[rng.random((n, k)) < 0.001] *= np.float32(10.0)
    elif dist == "t3":
        w = rng.standard_t(3, size=(n, k)).astype(np.float32)
    else:
        raise ValueError(dist)
    return w * s


def device_fp_weights(layer: int, proj: int, device):
    """fp32 (N, K) weights of one decoder projection, N(0, s^2) with s ~ U(0.01, 0.05),
    drawn on the GPU with torch (the stack's 5.2 GB would take long on the host)."""
    import torch
    _, k, n = PROJECTIONS[proj]
    rng = projection_rng(CFG_FPW, layer, proj, STREAM_SCALE)
    s = float(np.float32(rng.uniform(0.01, 0.05)))
    seed = int(np.random.SeedSequence([CFG_FPW, layer, proj, STREAM_W]).generate_state(
        1, np.uint64)[0] & np.uint64(2 ** 63 - 1))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((n, k), generator=g, device=device, dtype=torch.float32) * s


def small_problem(seed: int, m: int, n: int, k: int, dist: str = "normal",
                  p=None) -> dict:
    """Small seeded case for parity at sizes the oracle finishes in seconds."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000, seed, m, n, k])))
    if dist == "normal":
        x = rng.standard_normal((m, k), dtype=np.float32)
    elif dist == "t3":
        x = rng.standard_t(3, size=(m, k)).astype(np.float32)
    elif dist == "outlier":
        x = rng.standard_normal((m, k), dtype=np.float32)
        x[rng.random((m, k)) < 0.001] *= np.float32(20.0)
    else:
        raise ValueError(dist)
    w = ternary_weights(rng, n, k, p)
    return {"x": x, "w": w, "w_scale": np.float32(rng.uniform(0.01, 0.05)), "M": m, "N": n,
            "K": k}
