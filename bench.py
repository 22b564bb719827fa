"""Benchmark of the ternary-weight decoder matmul on one MI355X.

Headline workload: one decode step of the 28-layer, 1.5B-shaped decoder at M=1
(per layer QKV 1536->2048, O 1536->1536, gate+up 1536->17920, down 8960->1536;
327,548,928 bytes of 2-bit weights). A step quantizes the 112 activation
vectors (one grouped launch) and runs the 112 ternary GEMVs (one grouped
launch). Two copies of the weights alternate between steps so the 256 MB
on-package cache cannot hold them. value = packed weight bytes / step time.

Secondary workload (--prefill, on by default): long prefill, M=4096 tokens
through all 112 projections (per projection: quantize, then the MFMA GEMM),
reported as int8 TOPS = 2*M*N*K / time.

Beside them: the CPU oracle timed on the host's cores on a bounded sample
of the decode step (a reported baseline, not a target).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, TOPS
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_grouped_decode_step_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "ternary_weight_decoder_bt_amd", "csrc", "bt_kernels.hip")

METRIC = "ternary GEMV HBM GB/s (% of peak) + decode-step tokens/s; prefill int8 TOPS"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(per_launch_bytes: float):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernels changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# --------------------------------------------------------------- decode step

class DecodeStep:
    def __init__(self, torch, bt, dev, layers: int):
        self.torch, self.bt = torch, bt
        self.items_q, self.items = [], []
        self.w_bytes = 0
        self.alg_bytes = 0            # weights + q + y + scales per GEMV launch
        self.shapes = []
        wsets = ([], [])
        t0 = time.time()
        for layer in range(layers):
            for proj in range(len(synth.PROJECTIONS)):
                c = synth.decode_problem(layer, proj)
                m, k, n = c["M"], c["K"], c["N"]
                packed = torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev)
                wdev = bt.repack_ternary(packed, n, k)
                del packed
                wsets[0].append(wdev)
                wsets[1].append(wdev.clone())
                x = torch.from_numpy(c["x"]).to(dev)
                xq = torch.empty((m, k), dtype=torch.int8, device=dev)
                xs = torch.empty(m, dtype=torch.float32, device=dev)
                xsum = torch.empty(m, dtype=torch.int32, device=dev)
                y = torch.empty((m, n), dtype=torch.float32, device=dev)
                self.items_q.append((x, xq, xs, xsum))
                self.items.append({"xq": xq, "xscale": xs, "xsum": xsum, "n": n,
                                   "w_scale": c["w_scale"], "y": y})
                self.shapes.append((layer, proj, m, n, k))
                self.w_bytes += bt.packed_bytes(n, k)
                self.alg_bytes += bt.packed_bytes(n, k) + m * k + 4 * m * n + 8 * m
        self.qplan = bt.QuantPlan(self.items_q)
        self.mplans = [bt.MatmulPlan([dict(it, wdev=w) for it, w in zip(self.items, ws)])
                       for ws in wsets]
        self.wsets = wsets
        torch.cuda.synchronize()
        log(f"decode step ready: {len(self.items)} projections, {self.w_bytes} weight bytes, "
            f"setup {time.time() - t0:.1f}s")

    def step(self, i, ev=None):
        self.qplan.launch()
        if ev is not None:
            ev[0].record()
        self.mplans[i & 1].launch()
        if ev is not None:
            ev[1].record()

    def parity(self, idx_list):
        """Full oracle comparison of a few projections, untimed."""
        import oracle
        ok = True
        for idx in idx_list:
            layer, proj, m, n, k = self.shapes[idx]
            c = synth.decode_problem(layer, proj)
            ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
            it = self.items[idx]
            y = it["y"].cpu().numpy()
            ok &= np.array_equal(it["xq"].cpu().numpy(), ref["q"])
            ok &= np.array_equal(it["xscale"].cpu().numpy(), ref["d"])
            nz = ref["y"] != 0
            ok &= bool((y[~nz] == 0).all())
            ok &= bool((np.abs(y[nz] - ref["y"][nz]) <= 1e-6 * np.abs(ref["y"][nz])).all())
        return bool(ok)


# ----------------------------------------------------------- long prefill

def _pack_long_prefill(layer_proj):
    """Worker: long-prefill weights of one projection, packed on the host."""
    import ternary_weight_decoder_bt_amd as bt
    layer, proj = layer_proj
    return bt.pack_ternary(synth.long_prefill_problem(layer, proj, with_x=False)["w"])


def pack_long_prefill_weights(layers: int):
    """All long-prefill weights, drawn and packed in parallel host processes
    (before this process touches the GPU)."""
    import multiprocessing as mp
    jobs = [(layer, proj) for layer in range(layers) for proj in range(len(synth.PROJECTIONS))]
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with mp.get_context("spawn").Pool(workers) as pool:
        return pool.map(_pack_long_prefill, jobs, chunksize=1)


class LongPrefill:
    def __init__(self, torch, bt, dev, layers: int, m: int, packed_all):
        self.torch, self.bt = torch, bt
        self.probs = []
        self.ops = 0
        t0 = time.time()
        i = 0
        for layer in range(layers):
            for proj in range(len(synth.PROJECTIONS)):
                _, k, n = synth.PROJECTIONS[proj]
                packed = torch.from_numpy(packed_all[i].reshape(-1)).to(dev)
                i += 1
                wdev = bt.repack_ternary(packed, n, k)
                del packed
                x = synth.device_student_t3(m, k, synth.CFG_LONG, layer, proj, dev)
                s = synth.long_prefill_problem(layer, proj, m, with_weights=False,
                                               with_x=False)["w_scale"]
                p = {"x": x, "xq": torch.empty((m, k), dtype=torch.int8, device=dev),
                     "xs": torch.empty(m, dtype=torch.float32, device=dev),
                     "xsum": torch.empty(m, dtype=torch.int32, device=dev),
                     "y": torch.empty((m, n), dtype=torch.float32, device=dev),
                     "wdev": wdev, "n": n, "k": k, "s": s, "layer": layer, "proj": proj}
                self.probs.append(p)
                self.ops += 2 * m * n * k
        torch.cuda.synchronize()
        self.m = m
        log(f"long prefill ready: {len(self.probs)} projections, M={m}, "
            f"setup {time.time() - t0:.1f}s")

    def step(self, gemm_events=None):
        bt = self.bt
        for j, p in enumerate(self.probs):
            bt.quantize_act(p["x"], p["xq"], p["xs"], p["xsum"])
            if gemm_events is not None:
                gemm_events[j][0].record()
            bt.ternary_matmul(p["xq"], p["xs"], p["xsum"], p["wdev"], p["n"], p["s"], y=p["y"])
            if gemm_events is not None:
                gemm_events[j][1].record()

    def parity(self):
        """Sampled oracle comparison (rows and columns) on the first and last projection."""
        import oracle
        ok = True
        for p in (self.probs[0], self.probs[-1]):
            w = synth.long_prefill_problem(p["layer"], p["proj"], self.m, with_x=False)["w"]
            x = p["x"].cpu().numpy()
            q, d, _ = oracle.quantize_ref(x)
            ok &= np.array_equal(p["xq"].cpu().numpy(), q)
            y = p["y"].cpu().numpy()
            rows = np.array([0, 1, self.m // 2, self.m - 1])
            cols = np.array([0, 17, p["n"] // 2, p["n"] - 1])
            yr = oracle.dequant_ref(oracle.matmul_ref(q[rows], w, "f64"), d[rows], p["s"])
            yc = oracle.dequant_ref(oracle.matmul_ref(q, w[cols], "f64"), d, p["s"])
            for got, want in ((y[rows], yr), (y[:, cols], yc)):
                nz = want != 0
                ok &= bool((got[~nz] == 0).all())
                ok &= bool((np.abs(got[nz] - want[nz]) <= 1e-6 * np.abs(want[nz])).all())
        return bool(ok)


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(seconds: float):
    """The oracle as it stands (quantize, exact fp64-BLAS integer matmul,
    rescale) over the whole decode step, repeated until `seconds` (at least
    three passes); the median pass is reported."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    probs = [synth.decode_problem(layer, proj) for layer in range(synth.N_LAYERS)
             for proj in range(len(synth.PROJECTIONS))]
    w_bytes = sum(c["N"] * c["K"] // 4 for c in probs)
    passes, total = [], 0.0
    while len(passes) < 3 or total < seconds:
        t0 = time.perf_counter()
        for c in probs:
            oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
        passes.append(time.perf_counter() - t0)
        total += passes[-1]
    t = float(np.median(passes))
    return {"value": round(w_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole decode step (28 layers x 4 projections, M=1), {len(passes)} "
                      f"passes, median {t:.2f}s: oracle.forward_ref mode f64 (quantize + exact "
                      f"integer matmul through fp64 BLAS + rescale) on weights already unpacked "
                      f"to int8; value = packed weight bytes / pass time",
            "tokens_per_s": round(1.0 / t, 3),
            "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


# --------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=synth.N_LAYERS)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (5 times), to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each GPU would serve its own decode streams with replicated weights).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 4,
                          "copy_bytes_written_per_launch": dst.numel() * 4, "launches": 5}))
        return

    packed_prefill = None
    if not args.no_prefill:
        t0 = time.time()
        packed_prefill = pack_long_prefill_weights(args.layers)
        log(f"long-prefill weights drawn and packed on the host in {time.time() - t0:.1f}s")

    import torch

    import ternary_weight_decoder_bt_amd as bt
    bt.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")

    # ---- decode step (headline)
    ds = DecodeStep(torch, bt, dev, args.layers)
    ds.step(0)
    torch.cuda.synchronize()
    decode_ok = ds.parity([0, 1, 2, 3, len(ds.items) - 1])
    log(f"decode parity on sampled projections: {decode_ok}")
    for i in range(args.warmup):
        ds.step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        ds.step(i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    gemv_ms = [a.elapsed_time(b) for a, b in evs]
    gemv_avg_ms = float(np.mean(gemv_ms))
    value = ds.w_bytes / (ms_step * 1e-3) / 1e9
    achieved = ds.alg_bytes / (gemv_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(ds.alg_bytes)
    log(f"decode: {ms_step * 1e3:.1f} us/step, GEMV {gemv_avg_ms * 1e3:.1f} us "
        f"(p10 {np.percentile(gemv_ms, 10) * 1e3:.1f}, p90 {np.percentile(gemv_ms, 90) * 1e3:.1f}), "
        f"{value:.0f} GB/s, wall {t_wall:.2f}s")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded; ternary weights uniform over {-1,0,1}, x ~ N(0,1) with 0.1% x20; random-init, no checkpoint)",
        "config": {"workload": "decode step, 28-layer 1.5B-shaped decoder, M=1: per layer "
                               "qkv 1536->2048, o 1536->1536, gate_up 1536->17920, "
                               "down 8960->1536 (grouped quantize + grouped GEMV launch)",
                   "layers": args.layers, "M": 1, "weight_bytes_per_step": ds.w_bytes,
                   "weight_sets_alternating": 2},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(1e3 / ms_step, 1),
        "parity_ok": decode_ok,
        "roofline": {"bound": "hbm", "kernel": "gemv_grouped_kernel",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": ds.alg_bytes,
                     "avg_launch_ms": round(gemv_avg_ms, 5)},
    }
    del ds
    torch.cuda.empty_cache()

    # ---- long prefill (secondary)
    if not args.no_prefill:
        lp = LongPrefill(torch, bt, dev, args.layers, 4096, packed_prefill)
        del packed_prefill
        lp.step()
        torch.cuda.synchronize()
        pf_ok = lp.parity()
        gev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in lp.probs] for _ in range(args.prefill_steps)]
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for i in range(args.prefill_steps):
            lp.step(gev[i])
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / args.prefill_steps
        gemm_ms = float(np.mean([sum(a.elapsed_time(b) for a, b in g) for g in gev]))
        tops = lp.ops / (ms * 1e-3) / 1e12
        gemm_tops = lp.ops / (gemm_ms * 1e-3) / 1e12
        log(f"prefill: {ms:.3f} ms/stack ({tops:.0f} TOPS), GEMMs {gemm_ms:.3f} ms ({gemm_tops:.0f} TOPS)")
        out["prefill"] = {
            "workload": "long prefill, M=4096 tokens x 28 layers x 4 projections (quantize + GEMM each)",
            "int8_ops_per_stack": lp.ops, "ms_per_stack": round(ms, 4),
            "tops": round(tops, 2), "gemm_only_tops": round(gemm_tops, 2),
            "pct_of_int8_peak": round(100 * tops / I8_PEAK_TOPS, 2),
            "gemm_only_pct_of_int8_peak": round(100 * gemm_tops / I8_PEAK_TOPS, 2),
            "parity_ok": pf_ok, "steps": args.prefill_steps,
            "roofline": {"bound": "mfma", "kernel": "gemm_kernel", "achieved": round(gemm_tops, 2),
                         "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
                         "frac": round(gemm_tops / I8_PEAK_TOPS, 4)},
        }
        del lp
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
