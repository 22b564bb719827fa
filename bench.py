"""Benchmark of the ternary-weight decoder matmul on one MI355X.

Headline workload: one decode step of the 28-layer, 1.5B-shaped decoder at M=1
(per layer QKV 1536->2048, O 1536->1536, gate+up 1536->17920, down 8960->1536;
327,548,928 bytes of 2-bit weights). A step quantizes the 112 activation
vectors and runs the 112 ternary GEMVs in one launch (quantization fused into
the grouped GEMV); the same step as two launches (grouped quantize, grouped
GEMV) is reported beside it. Two copies of the weights alternate between steps
so the 256 MB on-package cache cannot hold them. value = packed weight bytes /
step time.

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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_decode_step_traffic.json")
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_long_prefill_traffic.json")
CSRC = os.path.join(ROOT, "ternary_weight_decoder_bt_amd", "csrc")
# the sources a kernel family's counters depend on (its kernels, shared helpers, host dispatch)
DECODE_SOURCES = ("bt_kernels.hip", "bt_device.h", "bt_internal.h", "bt_host.cpp")
GEMM_SOURCES = ("bt_gemm.hip", "bt_device.h", "bt_internal.h", "bt_host.cpp")

METRIC = "ternary GEMV HBM GB/s (% of peak) + decode-step tokens/s; prefill int8 TOPS"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(names) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_file(path, sources):
    """A committed counter summary, or None when its sources changed since the
    counters were taken."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_source_sha256_16") == source_hash(sources) else None


def measured_traffic(kernel: str):
    """HBM bytes per launch of the decode kernel `kernel` (or None)."""
    t = _traffic_file(TRAFFIC_FILE, DECODE_SOURCES)
    return None if t is None else t.get("kernels", {}).get(kernel, {}).get("hbm_bytes_per_launch")


def measured_gemm_traffic(form: str):
    """HBM bytes of the long-prefill stack's GEMMs in `form` ("grouped": one launch;
    "per_projection": 112 launches), or None."""
    t = _traffic_file(GEMM_TRAFFIC_FILE, GEMM_SOURCES)
    return None if t is None else t.get("forms", {}).get(form, {}).get("hbm_bytes_per_stack")


def capture_graph(torch, fn):
    """HIP graph of fn's launches (all on the capture stream). Warm-up runs on
    a side stream first, as graph capture requires."""
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


# --------------------------------------------------------------- decode step

class DecodeStep:
    """The 112 projections of one decode step, resident on the GPU.

    Headline path: one fused launch per step (bt_ternary_matmul_grouped with a
    plan whose descriptors carry the fp32 activations: quantization runs
    inside the GEMV). Context path: the same work as two launches (grouped
    quantize, then grouped GEMV on the quantized activations).
    """

    def __init__(self, torch, bt, dev, layers: int):
        self.torch, self.bt = torch, bt
        self.items_q, self.items, self.fitems = [], [], []
        self.packed = []              # canonical bytes on the device, for the repack timing
        self.w_bytes = 0
        self.alg_bytes = 0            # bytes the fused launch must move at least
        self.alg_bytes_gemv = 0       # bytes the unfused GEMV launch must move at least
        self.shapes = []
        wsets = ([], [])
        t0 = time.time()
        for layer in range(layers):
            for proj in range(len(synth.PROJECTIONS)):
                c = synth.decode_problem(layer, proj)
                m, k, n = c["M"], c["K"], c["N"]
                packed = torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev)
                wdev = bt.repack_ternary(packed, n, k)
                self.packed.append((packed, n, k))
                wsets[0].append(wdev)
                wsets[1].append(wdev.clone())
                x = torch.from_numpy(c["x"]).to(dev)
                xq = torch.empty((m, k), dtype=torch.int8, device=dev)
                xs = torch.empty(m, dtype=torch.float32, device=dev)
                xsum = torch.empty(m, dtype=torch.int32, device=dev)
                y = torch.empty((m, n), dtype=torch.float32, device=dev)
                self.items_q.append((x, xq, xs, xsum))
                base = {"xq": xq, "xscale": xs, "xsum": xsum, "n": n, "w_scale": c["w_scale"],
                        "y": y}
                self.items.append(base)
                self.fitems.append(dict(base, x=x))
                self.shapes.append((layer, proj, m, n, k))
                wb = bt.packed_bytes(n, k)
                self.w_bytes += wb
                # fused: read x, write q once, write y, write d and the row sum
                self.alg_bytes += wb + 4 * m * k + m * k + 4 * m * n + 8 * m
                # unfused GEMV: read q, d and the row sum, write y
                self.alg_bytes_gemv += wb + m * k + 4 * m * n + 8 * m
        self.qplan = bt.QuantPlan(self.items_q)
        self.mplans = [bt.MatmulPlan([dict(it, wdev=w) for it, w in zip(self.items, ws)])
                       for ws in wsets]
        self.fplans = [bt.MatmulPlan([dict(it, wdev=w) for it, w in zip(self.fitems, ws)])
                       for ws in wsets]
        self.wsets = wsets
        torch.cuda.synchronize()
        log(f"decode step ready: {len(self.items)} projections, {self.w_bytes} weight bytes, "
            f"setup {time.time() - t0:.1f}s")

    def time_repack(self, reps: int = 5):
        """The one-time device repack of the whole stack (112 launches), timed on its own.

        Two ways: the 112 single-tensor launches replayed from a HIP graph (so the time is
        the GPU's, not the host's launch rate), and one grouped launch over all of them.
        Rewrites weight set 0 with the same bytes. Returns {way: median ms per stack}.
        """
        torch, bt = self.torch, self.bt

        def run():
            for (packed, n, k), out in zip(self.packed, self.wsets[0]):
                bt.repack_ternary(packed, n, k, out=out)

        graph = capture_graph(torch, run)
        plan = bt.RepackPlan([(p, n, k, out) for (p, n, k), out in zip(self.packed,
                                                                           self.wsets[0])])
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        res = {}
        for name, fn in (("per_tensor_graph", graph.replay), ("grouped", plan.launch)):
            times = []
            for _ in range(reps + 1):
                start.record()
                fn()
                stop.record()
                torch.cuda.synchronize()
                times.append(start.elapsed_time(stop))
            res[name] = float(np.median(times[1:]))
        return res

    def step(self, i, ev=None):
        """One decode step as one fused launch (events, if given, bracket it)."""
        if ev is not None:
            ev[0].record()
        self.fplans[i & 1].launch()
        if ev is not None:
            ev[1].record()

    def chain(self, i, fused: bool):
        """One decode step as the dependent chain a decoder runs: the 112
        projections one after another on one stream, in decoder order (per
        layer qkv, o, gate_up, down), each a single call (fused: one launch that
        quantizes and multiplies; else bt_quantize_act then bt_ternary_matmul).
        Nothing overlaps: every launch waits for the one before it."""
        bt = self.bt
        for (x, xq, xs, xsum), it, w in zip(self.items_q, self.items, self.wsets[i & 1]):
            if fused:
                bt.ternary_matmul_fused(x, w, it["n"], it["w_scale"], y=it["y"], xq=xq,
                                        xscale=xs, xsum=xsum)
            else:
                bt.quantize_act(x, xq, xs, xsum)
                bt.ternary_matmul(xq, xs, xsum, w, it["n"], it["w_scale"], y=it["y"])

    def step_two_launch(self, i, ev=None):
        self.qplan.launch()
        if ev is not None:
            ev[0].record()
        self.mplans[i & 1].launch()
        if ev is not None:
            ev[1].record()

    def batched(self, m: int, steps: int, trials: int):
        """The same decode step for a batch of m tokens (m <= 16): the 112
        projections with m-row activations (seeded as the single-token step),
        the two weight sets alternating; quantization fused into the grouped
        GEMV, and as two launches (grouped quantize, grouped GEMV). Returns
        ({way: median ms per step}, parity of sampled projections)."""
        torch, bt = self.torch, self.bt
        import oracle
        dev = self.wsets[0][0].device
        fitems, qitems, gitems = [], [], []
        for (layer, proj, _m, n, k), it in zip(self.shapes, self.items):
            x = torch.from_numpy(synth.decode_problem(layer, proj, m, with_weights=False)["x"])
            x = x.to(dev)
            y = torch.full((m, n), float("nan"), device=dev)
            xq = torch.empty((m, k), dtype=torch.int8, device=dev)
            xs = torch.empty(m, dtype=torch.float32, device=dev)
            xsum = torch.empty(m, dtype=torch.int32, device=dev)
            fitems.append({"x": x, "n": n, "w_scale": it["w_scale"], "y": y})
            qitems.append((x, xq, xs, xsum))
            gitems.append({"xq": xq, "xscale": xs, "xsum": xsum, "n": n,
                           "w_scale": it["w_scale"], "y": y})
        fplans = [bt.MatmulPlan([dict(it, wdev=w) for it, w in zip(fitems, ws)])
                  for ws in self.wsets]
        qplan = bt.QuantPlan(qitems)
        gplans = [bt.MatmulPlan([dict(it, wdev=w) for it, w in zip(gitems, ws)])
                  for ws in self.wsets]
        ways = {"fused": lambda i: fplans[i & 1].launch(),
                "two_launch": lambda i: (qplan.launch(), gplans[i & 1].launch())}
        ok = True
        for fn in ways.values():
            for it in fitems:
                it["y"].fill_(float("nan"))
            fn(0)
            torch.cuda.synchronize()
            for idx in (0, 2, 3, len(fitems) - 1):
                layer, proj, _m, n, k = self.shapes[idx]
                c = synth.decode_problem(layer, proj, m)
                ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
                y = fitems[idx]["y"].cpu().numpy()
                nz = ref["y"] != 0
                ok &= bool((y[~nz] == 0).all())
                ok &= bool((np.abs(y[nz] - ref["y"][nz]) <= 1e-6 * np.abs(ref["y"][nz])).all())
        for fn in ways.values():
            for i in range(10):
                fn(i)
        torch.cuda.synchronize()
        times = {w: [] for w in ways}
        for _ in range(trials):
            for w, fn in ways.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for i in range(steps):
                    fn(i)
                b.record()
                torch.cuda.synchronize()
                times[w].append(a.elapsed_time(b) / steps)
        del fplans, gplans, qplan
        return {w: float(np.median(v)) for w, v in times.items()}, bool(ok)

    def clear_outputs(self):
        for it in self.items:
            it["y"].fill_(float("nan"))
            it["xq"].fill_(99)

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
            ok &= np.array_equal(it["xsum"].cpu().numpy(), ref["qsum"])
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
    """All long-prefill weights, drawn and packed on a pool of host threads (the
    C packing call and NumPy's bulk draws release the interpreter lock; threads
    start no process that could carry a profiler's preload)."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(layer, proj) for layer in range(layers) for proj in range(len(synth.PROJECTIONS))]
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        return list(pool.map(_pack_long_prefill, jobs))


class LongPrefill:
    def __init__(self, torch, bt, dev, layers: int, m: int, packed_all):
        self.torch, self.bt = torch, bt
        self.probs = []
        self.ops = 0
        self.alg_bytes = 0
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
                     "wdev": wdev, "n": n, "k": k, "s": s, "layer": layer, "proj": proj,
                     "ws": bt.new_workspace(m, n, k, dev)}
                self.probs.append(p)
                self.ops += 2 * m * n * k
                # int8 activations + 2-bit weights + fp32 output + scales and row sums
                self.alg_bytes += m * k + n * k // 4 + 4 * m * n + 8 * m
        torch.cuda.synchronize()
        self.m = m
        log(f"long prefill ready: {len(self.probs)} projections, M={m}, "
            f"setup {time.time() - t0:.1f}s")

    def build_grouped(self):
        """The same stack as two grouped launches: one quantization plan over the
        112 inputs, one GEMM plan over the 112 projections (each projection's
        workgroups walk its own output tiles), into separate output buffers."""
        torch, bt = self.torch, self.bt
        self.gitems = []
        for p in self.probs:
            m, k, n = self.m, p["k"], p["n"]
            self.gitems.append({
                "x": p["x"], "xq": torch.empty((m, k), dtype=torch.int8, device=p["x"].device),
                "xscale": torch.empty(m, dtype=torch.float32, device=p["x"].device),
                "xsum": torch.empty(m, dtype=torch.int32, device=p["x"].device),
                "y": torch.empty((m, n), dtype=torch.float32, device=p["x"].device),
                "wdev": p["wdev"], "n": n, "w_scale": p["s"]})
        self.gqplan = bt.QuantPlan([(g["x"], g["xq"], g["xscale"], g["xsum"])
                                    for g in self.gitems])
        self.ggplan = bt.MatmulPlan([{k_: g[k_] for k_ in ("xq", "xscale", "xsum", "y", "wdev",
                                                          "n", "w_scale")}
                                     for g in self.gitems])

    def step_grouped(self):
        self.gqplan.launch()
        self.ggplan.launch()

    def grouped_matches(self):
        """Every output of the grouped stack equals the per-projection stack's bit for
        bit (q, d, row sums and y; compared on the GPU)."""
        torch = self.torch
        ok = True
        for p, g in zip(self.probs, self.gitems):
            ok &= bool(torch.equal(p["xq"], g["xq"]) and torch.equal(p["xs"], g["xscale"]) and
                       torch.equal(p["xsum"], g["xsum"]) and torch.equal(p["y"], g["y"]))
        return ok

    def step(self):
        bt = self.bt
        for p in self.probs:
            bt.quantize_act(p["x"], p["xq"], p["xs"], p["xsum"])
            bt.ternary_matmul(p["xq"], p["xs"], p["xsum"], p["wdev"], p["n"], p["s"], y=p["y"],
                              workspace=p["ws"])

    def gemms(self):
        bt = self.bt
        for p in self.probs:
            bt.ternary_matmul(p["xq"], p["xs"], p["xsum"], p["wdev"], p["n"], p["s"], y=p["y"],
                              workspace=p["ws"])

    def time_shapes(self, reps: int = 20):
        """GEMM time of each of the four shapes (layer 0), each on its own: {name: (ms, TOPS)}."""
        torch, bt = self.torch, self.bt
        res = {}
        for p in self.probs[:len(synth.PROJECTIONS)]:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            call = lambda: bt.ternary_matmul(p["xq"], p["xs"], p["xsum"], p["wdev"], p["n"],
                                             p["s"], y=p["y"], workspace=p["ws"])
            call()
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            name = synth.PROJECTIONS[p["proj"]][0]
            res[name] = (ms, 2 * self.m * p["n"] * p["k"] / (ms * 1e-3) / 1e12)
        return res

    def time_epilogues(self, reps: int = 20):
        """Layer 0's gate_up with bias + ReLU and down with layer scale + residual add
        (the fused epilogues), each against the same GEMM without: {name: (ms, TOPS)}."""
        torch, bt = self.torch, self.bt
        res = {}
        for p, kind in ((self.probs[2], "bias_relu"), (self.probs[3], "scale_residual")):
            n = p["n"]
            vec = torch.linspace(-1, 1, n, device=p["y"].device)
            resid = torch.ones_like(p["y"])
            if kind == "bias_relu":
                kw = dict(bias=vec, relu=True)
            else:
                kw = dict(layer_scale=vec, residual=resid)
            name = synth.PROJECTIONS[p["proj"]][0]
            for tag, extra in (("plain", {}), (kind, kw)):
                call = lambda: bt.ternary_matmul(p["xq"], p["xs"], p["xsum"], p["wdev"], n, p["s"],
                                                 y=p["y"], workspace=p["ws"], **extra)
                call()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    call()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                res[f"{name}_{tag}"] = (ms, 2 * self.m * n * p["k"] / (ms * 1e-3) / 1e12)
        return res

    def time_activation_prologues(self, reps: int = 20):
        """Per-token quantization of layer 0's qkv (K=1536) and down (K=8960) inputs,
        plain and fused with RMS normalization: {name: (ms, GB/s)}."""
        torch, bt = self.torch, self.bt
        res = {}
        for p in (self.probs[0], self.probs[3]):
            m, k = self.m, p["k"]
            g = torch.linspace(0.5, 1.5, k, device=p["x"].device)
            for name, call, extra in (
                    ("quantize", lambda: bt.quantize_act(p["x"], p["xq"], p["xs"], p["xsum"]), 0),
                    ("rmsnorm_quantize", lambda: bt.rmsnorm_quantize(p["x"], g, 1e-6, p["xq"],
                                                                     p["xs"], p["xsum"]), 4 * k)):
                call()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    call()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                nbytes = 4 * m * k + m * k + 8 * m + extra
                res[f"{name}_M{m}_K{k}"] = (ms, nbytes / (ms * 1e-3) / 1e9)
        return res

    def parity_sampled(self):
        """Sampled oracle comparison (rows and columns) on the first and last projection.
        Every output of every projection is compared by tests/test_gpu_long_prefill_full.py;
        this check only guards the benchmark's own run."""
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


# ------------------------------------------------------- offline ternarization

def run_ternarize_stack(torch, bt, dev, layers: int, reps: int = 3):
    """The decode stack's 112 fp32 weight tensors (N(0, s^2), drawn on the GPU)
    ternarized (absmean) and packed on the device, replayed from a HIP graph.
    Parity: two tensors copied back and compared with the oracle byte for byte."""
    import oracle
    t0 = time.time()
    items = []
    alg = 0
    for layer in range(layers):
        for proj in range(len(synth.PROJECTIONS)):
            w = synth.device_fp_weights(layer, proj, dev)
            n, k = w.shape
            items.append((w, torch.empty(n * k // 4, dtype=torch.uint8, device=dev),
                          torch.empty(1, dtype=torch.float32, device=dev)))
            alg += 2 * 4 * n * k + n * k // 4 + 4     # two fp32 passes, packed bytes, scale
    need = max(bt.ternarize_workspace_bytes(*w.shape) for w, _, _ in items)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"ternarize: {len(items)} fp32 tensors ({sum(w.numel() for w, _, _ in items) * 4 / 1e9:.2f}"
        f" GB) ready in {time.time() - t0:.1f}s")

    def run():
        for w, p, sc in items:
            bt.ternarize(w, 1e-5, packed=p, scale=sc, workspace=ws)

    # the same stack as one grouped plan (two launches in all), into separate outputs
    gitems = [(w, torch.empty_like(p), torch.empty_like(sc)) for w, p, sc in items]
    plan = bt.TernarizePlan(gitems, 1e-5)
    run()
    plan.launch()
    torch.cuda.synchronize()
    ok = True
    for idx in (1, len(items) - 1):
        w, p, sc = items[idx]
        want_p, want_g = oracle.ternarize_pack_ref(w.cpu().numpy(), 1e-5)
        ok &= bool(np.array_equal(p.cpu().numpy(), want_p.reshape(-1)))
        ok &= bool(np.float32(sc.cpu().numpy()[0]) == want_g)
    grouped_same = all(bool(torch.equal(p, gp)) and bool(torch.equal(sc, gsc))
                       for (_, p, sc), (_, gp, gsc) in zip(items, gitems))

    def time_graph(fn):
        g = capture_graph(torch, fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(reps + 1):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del g
        return float(np.median(times[1:]))

    ms_single = time_graph(run)
    ms = time_graph(plan.launch)
    gbs = alg / (ms * 1e-3) / 1e9
    gbs_single = alg / (ms_single * 1e-3) / 1e9
    log(f"ternarize stack: grouped {ms:.3f} ms ({gbs:.0f} GB/s, {100 * gbs / HBM_PEAK_GBS:.1f}% "
        f"of HBM), single calls {ms_single:.3f} ms ({gbs_single:.0f} GB/s); parity {ok}, "
        f"grouped equals single calls: {grouped_same}")
    del plan, gitems, items, ws
    torch.cuda.empty_cache()
    return {"workload": "offline absmean ternarization + canonical packing of the decode "
                        "stack's 112 fp32 weight tensors (1.31e9 weights, N(0, s^2), "
                        "s ~ U(0.01, 0.05)), eps 1e-5, one grouped plan (two launches in all), "
                        "replayed from a HIP graph",
            "ms_per_stack": round(ms, 4), "algorithmic_bytes": alg,
            "gb_per_s": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "single_calls": {"workload": "the same stack as 112 bt_ternarize calls (two launches "
                                         "each), replayed from a HIP graph",
                             "ms_per_stack": round(ms_single, 4), "gb_per_s": round(gbs_single, 1),
                             "pct_of_hbm_peak": round(100 * gbs_single / HBM_PEAK_GBS, 2)},
            "grouped_equals_single_calls_bitwise": grouped_same,
            "parity_ok": ok}


# ------------------------------------------------- single-projection calls

def _rotating_copies(torch, wdev, min_bytes: int = 600 << 20):
    """Enough copies of one repacked weight tensor that cycling through them
    streams more than the 256 MB on-package cache holds."""
    n = max(2, -(-min_bytes // wdev.numel()))
    return [wdev] + [wdev.clone() for _ in range(n - 1)]


def _graph_us_per_call(torch, calls, reps: int = 5):
    """Median time per call of the `calls` (a list of closures, one launch sequence
    each), captured as one HIP graph and replayed `reps` times."""
    g = capture_graph(torch, lambda: [c() for c in calls])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps + 1):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / len(calls))
    del g
    return float(np.median(times[1:])) * 1e3


def run_single_projections(torch, bt, dev):
    """Single calls outside the grouped decode step:
    - one GEMV, M=1, K=N=1536 (x ~ N(0,1) seed 0, weights seed 1, scale 0.02), fused and
      two-launch;
    - the batched-decode remainder sweep: gate_up (1536->17920) and down (8960->1536) at
      M in {1,2,3,4,5,7,8,16}, GEMV on quantized activations;
    - one-layer prefill, M=512, the four projection shapes (quantize + GEMM each).
    Weights rotate over copies so they stream from HBM; calls replay from a HIP graph.
    Parity of each first output is checked against the oracle."""
    import oracle
    out = {}

    def close(got, want):
        nz = want != 0
        return bool((got[~nz] == 0).all() and
                    (np.abs(got[nz] - want[nz]) <= 1e-6 * np.abs(want[nz])).all())

    # ---- one GEMV, M=1, 1536 x 1536
    c = synth.config0()
    ref = oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
    packed = torch.from_numpy(bt.pack_ternary(c["w"]).reshape(-1)).to(dev)
    ws_ = _rotating_copies(torch, bt.repack_ternary(packed, c["N"], c["K"]))
    x = torch.from_numpy(c["x"]).to(dev)
    y = torch.empty((1, c["N"]), dtype=torch.float32, device=dev)
    xq = torch.empty((1, c["K"]), dtype=torch.int8, device=dev)
    xs = torch.empty(1, dtype=torch.float32, device=dev)
    xsum = torch.empty(1, dtype=torch.int32, device=dev)
    wb = bt.packed_bytes(c["N"], c["K"])
    ok = True
    bt.ternary_matmul_fused(x, ws_[0], c["N"], c["w_scale"], y=y, xq=xq, xscale=xs, xsum=xsum)
    torch.cuda.synchronize()
    ok &= close(y.cpu().numpy(), ref["y"]) and np.array_equal(xq.cpu().numpy(), ref["q"])
    y.fill_(float("nan"))
    bt.quantize_act(x, xq, xs, xsum)
    bt.ternary_matmul(xq, xs, xsum, ws_[0], c["N"], c["w_scale"], y=y)
    torch.cuda.synchronize()
    ok &= close(y.cpu().numpy(), ref["y"])
    fused_us = _graph_us_per_call(torch, [
        (lambda w=w: bt.ternary_matmul_fused(x, w, c["N"], c["w_scale"], y=y)) for w in ws_])
    gemv_us = _graph_us_per_call(torch, [
        (lambda w=w: bt.ternary_matmul(xq, xs, xsum, w, c["N"], c["w_scale"], y=y)) for w in ws_])
    two_us = _graph_us_per_call(torch, [
        (lambda w=w: (bt.quantize_act(x, xq, xs, xsum),
                      bt.ternary_matmul(xq, xs, xsum, w, c["N"], c["w_scale"], y=y)))
        for w in ws_])
    # all bytes: the GEMV alone reads the weights, the int8 row, its scale and row sum and
    # writes y; fused it reads the fp32 row instead; two launches also write and re-read q
    k_, n_ = c["K"], c["N"]
    all_gemv = wb + k_ + 8 + 4 * n_
    all_fused = wb + 4 * k_ + 4 * n_
    all_two = wb + 4 * k_ + 2 * (k_ + 8) + 4 * n_
    out["gemv_1536x1536_M1"] = {
        "workload": "one ternary GEMV, M=1, K=N=1536, weights streamed from HBM "
                    f"({len(ws_)} rotating copies), calls replayed from a HIP graph",
        "weight_bytes": wb, "parity_ok": bool(ok),
        "fused_us": round(fused_us, 3), "two_launch_us": round(two_us, 3),
        "gemv_only_us": round(gemv_us, 3),
        "gemv_only_weight_gb_per_s": round(wb / (gemv_us * 1e-6) / 1e9, 1),
        "fused_weight_gb_per_s": round(wb / (fused_us * 1e-6) / 1e9, 1),
        "all_bytes": {"gemv_only": all_gemv, "fused": all_fused, "two_launch": all_two},
        "gemv_only_all_bytes_gb_per_s": round(all_gemv / (gemv_us * 1e-6) / 1e9, 1),
        "fused_all_bytes_gb_per_s": round(all_fused / (fused_us * 1e-6) / 1e9, 1),
        "two_launch_all_bytes_gb_per_s": round(all_two / (two_us * 1e-6) / 1e9, 1),
        "gemv_only_pct_of_hbm_peak": round(100 * all_gemv / (gemv_us * 1e-6) / 1e9 /
                                           HBM_PEAK_GBS, 2)}
    log(f"single GEMV 1536x1536: fused {fused_us:.2f} us, two-launch {two_us:.2f} us, "
        f"GEMV alone {gemv_us:.2f} us ({wb / (gemv_us * 1e-6) / 1e9:.0f} GB/s); parity {ok}")
    del ws_, packed

    # ---- batched-decode remainder sweep
    sweep = {}
    for name in ("gate_up", "down"):
        c1 = synth.decode_remainder_problem(name, 1)
        n, k = c1["N"], c1["K"]
        packed = torch.from_numpy(bt.pack_ternary(c1["w"]).reshape(-1)).to(dev)
        ws_ = _rotating_copies(torch, bt.repack_ternary(packed, n, k))
        wb = bt.packed_bytes(n, k)
        row = {}
        for m in synth.REMAINDER_MS:
            cm = synth.decode_remainder_problem(name, m)
            x = torch.from_numpy(cm["x"]).to(dev)
            q = bt.quantize_act(x)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            wsp = bt.new_workspace(m, n, k, dev)
            bt.ternary_matmul(*q, ws_[0], n, cm["w_scale"], y=y, workspace=wsp)
            torch.cuda.synchronize()
            cols = np.array([0, 1, n // 2, n - 1])
            want = oracle.dequant_ref(oracle.matmul_ref(q[0].cpu().numpy(), cm["w"][cols], "f64"),
                                      q[1].cpu().numpy(), cm["w_scale"])
            good = close(y.cpu().numpy()[:, cols], want)
            us = _graph_us_per_call(torch, [
                (lambda w=w: bt.ternary_matmul(*q, w, n, cm["w_scale"], y=y, workspace=wsp))
                for w in ws_])
            alg = wb + m * k + 4 * m * n + 8 * m
            row[f"M{m}"] = {"us": round(us, 3), "gb_per_s": round(alg / (us * 1e-6) / 1e9, 1),
                            "pct_of_hbm_peak": round(100 * alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                                     2),
                            "parity_ok": good}
        sweep[name] = row
        log(f"remainder sweep {name}: " + ", ".join(
            f"M={m} {row[f'M{m}']['us']:.1f}us/{row[f'M{m}']['gb_per_s']:.0f}GB/s"
            for m in synth.REMAINDER_MS))
        del ws_, packed
    out["remainder_sweep"] = {
        "workload": "gate_up 1536->17920 and down 8960->1536 at M in {1,2,3,4,5,7,8,16}, "
                    "GEMV on quantized activations, weights streamed from HBM, calls replayed "
                    "from a HIP graph; GB/s = (weights + activations + output) / time",
        "shapes": sweep}

    # ---- one-layer prefill, M=512
    pre, tot_ops, tot_us, gemm_us_tot = {}, 0, 0.0, 0.0
    layer = []
    for proj in range(len(synth.PROJECTIONS)):
        cp = synth.prefill_problem(proj)
        m, n, k = cp["M"], cp["N"], cp["K"]
        packed = torch.from_numpy(bt.pack_ternary(cp["w"]).reshape(-1)).to(dev)
        wdev = bt.repack_ternary(packed, n, k)
        x = torch.from_numpy(cp["x"]).to(dev)
        q = bt.quantize_act(x)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        wsp = bt.new_workspace(m, n, k, dev)
        bt.ternary_matmul(*q, wdev, n, cp["w_scale"], y=y, workspace=wsp)
        torch.cuda.synchronize()
        rows = np.array([0, 1, m // 2, m - 1])
        qn = q[0].cpu().numpy()
        want = oracle.dequant_ref(oracle.matmul_ref(qn[rows], cp["w"], "f64"),
                                  q[1].cpu().numpy()[rows], cp["w_scale"])
        good = close(y.cpu().numpy()[rows], want)
        reps = 20
        gemm_us = _graph_us_per_call(torch, [
            (lambda: bt.ternary_matmul(*q, wdev, n, cp["w_scale"], y=y, workspace=wsp))] * reps)
        both_us = _graph_us_per_call(torch, [
            (lambda: (bt.quantize_act(x, *q),
                      bt.ternary_matmul(*q, wdev, n, cp["w_scale"], y=y, workspace=wsp)))] * reps)
        ops = 2 * m * n * k
        tot_ops += ops
        tot_us += both_us
        gemm_us_tot += gemm_us
        pre[cp["name"]] = {"M": m, "N": n, "K": k, "gemm_us": round(gemm_us, 2),
                           "gemm_tops": round(ops / (gemm_us * 1e-6) / 1e12, 1),
                           "quantize_plus_gemm_us": round(both_us, 2), "parity_ok": good}
        layer.append({"m": m, "n": n, "k": k, "s": cp["w_scale"], "x": x, "wdev": wdev, "y": y,
                      "xq": torch.empty((m, k), dtype=torch.int8, device=dev),
                      "xs": torch.empty(m, dtype=torch.float32, device=dev),
                      "xsum": torch.empty(m, dtype=torch.int32, device=dev),
                      "y2": torch.empty((m, n), dtype=torch.float32, device=dev), "ws": wsp})
        del packed, q
    # the same layer with its four independent projections overlapped: one grouped
    # quantization launch and one grouped GEMM launch (down, 24 tiles over K = 8960,
    # split there into K ranges whose partial sums a reduce launch adds)
    qplan = bt.QuantPlan([(L_["x"], L_["xq"], L_["xs"], L_["xsum"]) for L_ in layer])
    gplan = bt.MatmulPlan([{"xq": L_["xq"], "xscale": L_["xs"], "xsum": L_["xsum"],
                            "wdev": L_["wdev"], "n": L_["n"], "w_scale": L_["s"], "y": L_["y2"]}
                           for L_ in layer])

    def grouped_layer():
        qplan.launch()
        gplan.launch()

    grouped_layer()
    torch.cuda.synchronize()
    grouped_same = all(bool(torch.equal(L_["y"], L_["y2"])) for L_ in layer)
    grouped_us = _graph_us_per_call(torch, [grouped_layer] * 20)
    del qplan, gplan, layer
    out["prefill_M512_one_layer"] = {
        "workload": "one layer's four projections at M=512 (weights P(-1,0,1) = 0.3/0.4/0.3, "
                    "x ~ N(0,1)), quantize + GEMM each, replayed from a HIP graph "
                    "(L2-warm: each call reuses one weight tensor)",
        "shapes": pre, "ms_per_layer": round(tot_us * 1e-3, 4),
        "tops": round(tot_ops / (tot_us * 1e-6) / 1e12, 1),
        "gemm_only_tops": round(tot_ops / (gemm_us_tot * 1e-6) / 1e12, 1),
        "pct_of_int8_peak": round(100 * tot_ops / (tot_us * 1e-6) / 1e12 / I8_PEAK_TOPS, 2),
        "grouped": {"workload": "the four independent projections overlapped: one grouped "
                                "quantization launch, one grouped GEMM launch (down split into "
                                "K ranges, plus the launch that adds their partial sums); "
                                "replayed from a HIP graph",
                    "us_per_layer": round(grouped_us, 2),
                    "tops": round(tot_ops / (grouped_us * 1e-6) / 1e12, 1),
                    "pct_of_int8_peak": round(100 * tot_ops / (grouped_us * 1e-6) / 1e12 /
                                              I8_PEAK_TOPS, 2),
                    "matches_per_projection_bitwise": grouped_same}}
    log(f"prefill M=512 one layer: {tot_us:.1f} us ({tot_ops / (tot_us * 1e-6) / 1e12:.0f} TOPS), "
        f"GEMMs {gemm_us_tot:.1f} us; " + ", ".join(
            f"{k_} {v['gemm_tops']:.0f}" for k_, v in pre.items()) +
        f"; grouped {grouped_us:.1f} us ({tot_ops / (grouped_us * 1e-6) / 1e12:.0f} TOPS), "
        f"matches per-projection: {grouped_same}")
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ CPU baseline

# The tokenizer's ConvNeXt stages ("VibeVoice-ASR-BitNet Technical Report",
# section 2.2.1, Table 1: channels D and sequence length L for 20 s of audio);
# each block's FFN is D -> 4D -> D, run here as two I8_S GEMMs with M = L.
VAE_STAGES = ((32, 480000), (64, 240000), (128, 120000), (256, 30000), (512, 6000),
              (1024, 1200), (2048, 150))


def run_remainder_for_counters(torch, bt, dev, reps: int):
    """The remainder sweep's points (gate_up, then down, each M in order), each
    launched `reps` times eagerly on rotating weight copies, for a counter pass
    of the profiler: every call's GEMV launches in order, so the n-th group of
    `reps` gemv_kernel dispatches is the n-th point (a split call adds one
    reduce launch, named otherwise). Prints the point order as JSON."""
    points = []
    for name in ("gate_up", "down"):
        c1 = synth.decode_remainder_problem(name, 1)
        n, k = c1["N"], c1["K"]
        packed = torch.from_numpy(bt.pack_ternary(c1["w"]).reshape(-1)).to(dev)
        ws_ = _rotating_copies(torch, bt.repack_ternary(packed, n, k))
        for m in synth.REMAINDER_MS:
            cm = synth.decode_remainder_problem(name, m)
            q = bt.quantize_act(torch.from_numpy(cm["x"]).to(dev))
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            wsp = bt.new_workspace(m, n, k, dev)
            torch.cuda.synchronize()
            for i in range(reps):
                bt.ternary_matmul(*q, ws_[(7 * i + 1) % len(ws_)], n, cm["w_scale"], y=y,
                                  workspace=wsp)
            torch.cuda.synchronize()
            points.append({"shape": name, "M": m, "N": n, "K": k,
                           "alg_bytes": bt.packed_bytes(n, k) + m * k + 4 * m * n + 8 * m})
        del ws_, packed
    print(json.dumps({"remainder_points": points, "reps": reps}), flush=True)


def run_i8s_tokenizer_ffn(torch, bt, dev, reps: int = 10):
    """Time the I8_S GEMMs of the tokenizer's FFN layers (synthetic int8 codes and
    weights). Returns {stage: {...}} and the aggregate."""
    out = {}
    tot_ops, tot_ms, tot_bytes = 0, 0.0, 0
    gen = torch.Generator(device=dev).manual_seed(7)
    for st, (d, L) in enumerate(VAE_STAGES):
        row = {}
        for name, (n, k) in (("up", (4 * d, d)), ("down", (d, 4 * d))):
            xq = torch.randint(-127, 128, (L, k), dtype=torch.int8, device=dev, generator=gen)
            xs = torch.rand(L, device=dev, generator=gen) * 0.01 + 0.001
            w8 = torch.randint(-128, 128, (n, k), dtype=torch.int8, device=dev, generator=gen)
            wdev = bt.repack_int8(w8)
            y = torch.empty((L, n), dtype=torch.float32, device=dev)
            need = bt.int8_matmul_workspace_bytes(L, n, k)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev) if need else None
            bt.int8_matmul(xq, xs, wdev, n, 0.01, y=y, workspace=ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                bt.int8_matmul(xq, xs, wdev, n, 0.01, y=y, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            ops = 2 * L * n * k
            nbytes = L * k + n * k + 4 * L * n + 4 * L
            row[name] = {"M": L, "N": n, "K": k, "us": round(ms * 1e3, 2),
                         "tops": round(ops / (ms * 1e-3) / 1e12, 1),
                         "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "bound": "hbm" if ops / nbytes < I8_PEAK_TOPS / HBM_PEAK_GBS * 1e3
                                  else "mfma"}
            tot_ops += ops
            tot_ms += ms
            tot_bytes += nbytes
            del xq, xs, w8, wdev, y
        out[f"stage{st}_D{d}_L{L}"] = row
        log(f"i8s stage {st} (D={d}, L={L}): up {row['up']['tops']} TOPS / "
            f"{row['up']['gb_per_s']} GB/s, down {row['down']['tops']} TOPS / "
            f"{row['down']['gb_per_s']} GB/s")
    torch.cuda.empty_cache()
    return {"workload": "I8_S GEMMs of the tokenizer's FFN layers (D -> 4D -> D, M = L) for "
                        "the 7 stages of a 20 s input, synthetic int8 codes and weights, "
                        "fp32 output",
            "stages": out, "total_us": round(tot_ms * 1e3, 1),
            "tops": round(tot_ops / (tot_ms * 1e-3) / 1e12, 1),
            "gb_per_s": round(tot_bytes / (tot_ms * 1e-3) / 1e9, 1)}


def run_ceilings(torch, dev):
    """What the part itself reaches, for the rooflines' denominators: the
    v_mfma_i32_16x16x64_i8 issue rate (operands in registers, eight
    independent chains per wave, 2 and 4 waves per SIMD) with the shader
    clock it ran at, and a plain streaming read by size (each read takes a
    fresh window of a 2 GiB buffer, so no size is served from the 256 MB
    last-level cache; launches are back to back, so the smallest sizes
    include the gap between launches)."""
    from ternary_weight_decoder_bt_amd import ceilings as cl
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wall_khz = cl.wall_clock_khz(dev.index or 0)
    clocks = torch.zeros(4, dtype=torch.int64, device=dev)
    iters = 16384
    mfma = {}
    for waves_per_simd in (2, 4):
        blocks = cus * waves_per_simd   # 4 waves per workgroup, one per SIMD
        out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        cl.mfma_i8_issue(blocks, iters, 1, 1, out, clocks, stream)   # warm-up
        times, ghz = [], []
        for _ in range(5):
            out.fill_(0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            cl.mfma_i8_issue(blocks, iters, 1, 1, out, clocks, stream)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
            c = clocks.cpu().tolist()
            if wall_khz > 0 and c[3] > c[1]:
                ghz.append((c[2] - c[0]) / ((c[3] - c[1]) / (wall_khz * 1e3)) / 1e9)
        ok = bool((out == cl.expected_issue_sum(iters, 1, 1)).all().item())
        ms = float(np.median(times))
        ops = blocks * 4 * iters * 8 * 2 * 16 * 16 * 64
        tops = ops / (ms * 1e-3) / 1e12
        clk = float(np.median(ghz)) if ghz else None
        mfma[f"{waves_per_simd}_waves_per_simd"] = {
            "tops": round(tops, 1), "ms": round(ms, 4), "checksum_ok": ok,
            "shader_clock_ghz": None if clk is None else round(clk, 3),
            "ops_per_cu_per_cycle": None if not clk else round(tops * 1e12 / cus / (clk * 1e9), 1)}
    best = max(mfma.values(), key=lambda v: v["tops"])
    per_cycle = best["ops_per_cu_per_cycle"]
    res = {"compute_units": cus, "wall_clock_khz": wall_khz,
           "mfma_i32_16x16x64_i8": mfma,
           "int8_peak_tops_measured": best["tops"],
           "int8_peak_tops_derived_at_2p4ghz": None if not per_cycle
           else round(per_cycle * cus * 2.4e9 / 1e12, 1),
           "int8_peak_tops_published": I8_PEAK_TOPS}

    buf_bytes = 2 << 30
    buf = torch.empty(buf_bytes // 4, dtype=torch.int32, device=dev)
    buf.random_()
    reads = []
    xor_out = torch.empty(cus * 32 * 16, dtype=torch.int32, device=dev)
    for mb in (1, 4, 16, 64, 256, 1024, 2048):
        nbytes = mb << 20
        windows = buf_bytes // nbytes
        reps = max(3, min(64, (512 << 20) // nbytes))
        base = buf.data_ptr()
        best = None
        # 8 and 32 workgroups per compute unit (the more the better beyond a
        # few hundred MB); the faster is reported
        for per_cu in (8, 32):
            blocks = max(1, min(cus * per_cu, nbytes // (256 * 16 * 8)))
            cl.stream_read(base, nbytes, blocks, xor_out, stream)   # warm-up
            trials = []
            w = 1
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(reps):
                    cl.stream_read(base + (w % windows) * nbytes, nbytes, blocks, xor_out, stream)
                    w += 1
                b.record()
                torch.cuda.synchronize()
                trials.append(a.elapsed_time(b) / reps)
            ms = float(np.median(trials))
            if best is None or ms < best[0]:
                best = (ms, blocks)
        ms, blocks = best
        reads.append({"mb": mb, "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                      "us_per_read": round(ms * 1e3, 2), "workgroups": blocks,
                      "fresh_windows": windows > 1})
    # the kernel read every byte: XOR of its outputs == XOR of the first 1 MiB
    cl.stream_read(base, 1 << 20, 64, xor_out, stream)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(xor_out[:64 * 16].cpu().numpy().view(np.uint32).reshape(-1, 4))
    want = np.bitwise_xor.reduce(buf[: (1 << 20) // 4].cpu().numpy().view(np.uint32).reshape(-1, 4))
    res["stream_read"] = reads
    res["stream_read_checksum_ok"] = bool(np.array_equal(got, want))
    res["stream_read_peak_gb_per_s"] = max(r["gb_per_s"] for r in reads)
    res["hbm_peak_gb_per_s_published"] = HBM_PEAK_GBS
    del buf
    torch.cuda.empty_cache()
    return res


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        return 1


def _timed(fn, runs: int = 3, warm: int = 1):
    """Median wall time of `runs` calls after `warm` untimed ones, and every run."""
    for _ in range(warm):
        fn()
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), ts


def _one_core():
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def cpu_baseline_configs(oracle):
    """The oracle on the other workloads, each on a bounded sample (sizes stated):
    brute int64 dot products on one thread for the single GEMV, one layer of the
    decode step and the remainder sweep; exact fp64 BLAS on all cores and on one
    core for the prefills. Timed
    region: quantize + integer matmul + rescale (oracle.forward_ref) on weights
    already unpacked to int8."""
    out = {}
    # single GEMV, M=1, K=N=1536: brute, one thread
    c = synth.config0()
    with _one_core():
        t, ts = _timed(lambda: oracle.forward_ref(c["x"], c["w"], c["w_scale"], "int64"), 5)
    wb = c["N"] * c["K"] // 4
    allb = wb + 4 * c["K"] + c["K"] + 4 * c["N"] + 8
    out["single_gemv_1536x1536_M1"] = {
        "mode": "brute (int64 dot products), 1 thread", "cores": 1, "us": round(t * 1e6, 1),
        "weight_gb_per_s": round(wb / t / 1e9, 4), "all_bytes_gb_per_s": round(allb / t / 1e9, 4),
        "sample": "the whole workload, median of 5 runs after 1 warm-up"}
    # decode step: brute, one thread, on layer 0's four projections
    layer = [synth.decode_problem(0, proj) for proj in range(len(synth.PROJECTIONS))]
    with _one_core():
        t, _ = _timed(lambda: [oracle.forward_ref(c["x"], c["w"], c["w_scale"], "int64")
                               for c in layer], 3)
    lb = sum(c["N"] * c["K"] // 4 for c in layer)
    out["decode_step_layer0_brute"] = {
        "mode": "brute (int64 dot products), 1 thread", "cores": 1, "ms": round(t * 1e3, 2),
        "weight_gb_per_s": round(lb / t / 1e9, 4),
        "tokens_per_s_28_layers": round(1.0 / (28 * t), 3),
        "sample": "layer 0's four projections (one of the 28 layers of the decode step), median "
                  "of 3 after 1 warm-up"}
    # remainder sweep: brute, one thread, every point once
    sweep = {}
    with _one_core():
        for name in ("gate_up", "down"):
            w = synth.decode_remainder_problem(name, 1)["w"]
            n, k = w.shape
            row = {}
            for m in synth.REMAINDER_MS:
                cm = synth.decode_remainder_problem(name, m)
                t, _ = _timed(lambda: oracle.forward_ref(cm["x"], w, cm["w_scale"], "int64"), 1,
                              1 if m == 1 else 0)
                row[f"M{m}"] = {"us": round(t * 1e6, 1),
                                "gb_per_s": round((n * k // 4 + m * k + 4 * m * n + 8 * m)
                                                  / t / 1e9, 4)}
            sweep[name] = row
    out["remainder_sweep"] = {"mode": "brute (int64 dot products), 1 thread", "cores": 1,
                              "sample": "every (shape, M) point once, after one warm-up at M=1",
                              "shapes": sweep}
    # prefill M=512, one layer: exact fp64 BLAS, all cores and one core
    probs = [synth.prefill_problem(p) for p in range(len(synth.PROJECTIONS))]
    ops = sum(2 * c["M"] * c["N"] * c["K"] for c in probs)
    run = lambda: [oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64") for c in probs]
    t_all, _ = _timed(run)
    with _one_core():
        t_one, _ = _timed(run)
    out["prefill_M512_one_layer"] = {
        "mode": "exact fp64 BLAS", "cores_all": _blas_threads(),
        "tops_all_cores": round(ops / t_all / 1e12, 5), "tops_one_core": round(ops / t_one / 1e12, 5),
        "ms_all_cores": round(t_all * 1e3, 1), "ms_one_core": round(t_one * 1e3, 1),
        "sample": "the whole workload (4 projections at M=512), median of 3 after 1 warm-up"}
    # long prefill: the first 512 token rows of layer 0's four projections
    rows = 512
    probs = [synth.long_prefill_problem(0, p, rows) for p in range(len(synth.PROJECTIONS))]
    ops = sum(2 * rows * c["N"] * c["K"] for c in probs)
    run = lambda: [oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64") for c in probs]
    t_all, _ = _timed(run)
    with _one_core():
        t_one, _ = _timed(run)
    out["long_prefill"] = {
        "mode": "exact fp64 BLAS", "cores_all": _blas_threads(),
        "tops_all_cores": round(ops / t_all / 1e12, 5), "tops_one_core": round(ops / t_one / 1e12, 5),
        "ms_all_cores": round(t_all * 1e3, 1), "ms_one_core": round(t_one * 1e3, 1),
        "sample": f"layer 0's four projections on {rows} of the 4096 token rows (Student-t(3) "
                  f"activations, weights P = 0.2/0.6/0.2), {ops} int8 ops per pass, median of "
                  f"3 after 1 warm-up"}
    return out


def cpu_baseline(seconds: float):
    """The oracle as it stands (quantize, exact fp64-BLAS integer matmul,
    rescale) over the whole decode step, repeated until `seconds` (at least
    three passes); the median pass is reported. The other workloads follow on
    bounded samples (cpu_baseline_configs)."""
    import oracle
    threads = _blas_threads()
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
    # the same on one core, over one layer (the four projections), and the
    # oracle's unpacking of that layer's canonical 2-bit bytes, timed apart
    layer = probs[:len(synth.PROJECTIONS)]
    layer_bytes = sum(c["N"] * c["K"] // 4 for c in layer)
    one_core = None
    try:
        with _one_core():
            tl, _ = _timed(lambda: [oracle.forward_ref(c["x"], c["w"], c["w_scale"], "f64")
                                    for c in layer], 3, 0)
        one_core = {"value": round(layer_bytes / tl / 1e9, 4), "unit": "GB/s",
                    "cores": 1, "sample": "layer 0's four projections, median of 3 passes"}
    except Exception:  # noqa: BLE001
        pass
    packed = [oracle.pack_ref(c["w"]) for c in layer]
    tu, _ = _timed(lambda: [oracle.unpack_ref(pk, c["K"]) for c, pk in zip(layer, packed)], 3, 0)
    unpack = {"value": round(layer_bytes / tu / 1e9, 4),
              "unit": "GB/s of packed bytes", "cores": 1,
              "sample": "oracle.unpack_ref over layer 0's four projections, median of 3 passes"}
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    configs = None
    try:
        configs = cpu_baseline_configs(oracle)
    except Exception as e:  # noqa: BLE001
        log(f"cpu baseline on the other workloads failed: {e!r}")
    return {"value": round(w_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole decode step (28 layers x 4 projections, M=1), {len(passes)} "
                      f"passes, median {t:.2f}s: oracle.forward_ref mode f64 (quantize + exact "
                      f"integer matmul through fp64 BLAS + rescale) on weights already unpacked "
                      f"to int8; value = packed weight bytes / pass time",
            "tokens_per_s": round(1.0 / t, 3),
            "pass_s_p10_p50_p90": [round(float(np.percentile(passes, q)), 4) for q in (10, 50, 90)],
            "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model,
            "one_core": one_core,
            "unpack": unpack,
            "configs": configs}


def clock_under_load(torch, bt, seconds: float):
    """The shader clock while the long-prefill stack's grouped GEMM launch (112
    projections, M=4096, random int8 activations and ternary codes) runs back to
    back for `seconds`: `rocm-smi --showclocks` is read every half second from a
    host thread (a read-only query). The published int8 peak is stated at 2.4 GHz;
    under this load the part runs lower."""
    import re
    import subprocess
    import threading
    dev = torch.device("cuda:0")
    m = 4096
    g = torch.Generator(device=dev).manual_seed(1)
    xs = torch.rand(m, device=dev, generator=g) * 0.01
    xsum = torch.randint(-1000, 1000, (m,), dtype=torch.int32, device=dev, generator=g)
    items = []
    for _layer in range(synth.N_LAYERS):
        for _, k, n in synth.PROJECTIONS:
            w = torch.randint(0, 255, (bt.repacked_bytes(n, k),), dtype=torch.uint8, device=dev,
                              generator=g) & 0x55        # codes 0 and 1: weights -1 and 0
            items.append({"xq": torch.randint(-127, 128, (m, k), dtype=torch.int8, device=dev,
                                              generator=g),
                          "xscale": xs, "xsum": xsum, "wdev": w, "n": n, "w_scale": 0.02,
                          "y": torch.empty((m, n), device=dev)})
    ops = sum(2 * m * it["n"] * it["xq"].shape[1] for it in items)
    plan = bt.MatmulPlan(items)
    plan.launch()
    torch.cuda.synchronize()
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                                     timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            mhz = [int(v) for v in re.findall(r"sclk clock level: \S+: \((\d+)Mhz\)", txt)]
            if mhz:
                samples.append(mhz[0])
            stop.wait(0.5)

    th = threading.Thread(target=sample, daemon=True)
    started = False
    t0 = time.time()
    launches_ms = []
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while time.time() - t0 < seconds:
        a.record()
        for _ in range(20):
            plan.launch()
        b.record()
        torch.cuda.synchronize()
        launches_ms.append(a.elapsed_time(b) / 20)
        if not started and time.time() - t0 > 1.0:   # sample once the load is steady
            th.start()
            started = True
        log(f"clock under load: {time.time() - t0:.1f}s, {launches_ms[-1]:.3f} ms per launch, "
            f"sclk samples {samples[-3:]}")
    stop.set()
    if started:
        th.join(timeout=15)
    ms = float(np.median(launches_ms))
    return {"workload": "the long-prefill stack's grouped GEMM launch back to back, random int8 "
                        "operands", "seconds": seconds, "ms_per_launch_median": round(ms, 4),
            "tops": round(ops / (ms * 1e-3) / 1e12, 1), "sclk_mhz_samples": samples,
            "sclk_mhz_median": float(np.median(samples)) if samples else None,
            "int8_peak_tops_at_that_clock": round(5000.0 * float(np.median(samples)) / 2400.0, 1)
            if samples else None}


def run_batched_decode(ds, out, args):
    """The decode step for a batch of 16 tokens, fused and as two launches."""
    b_ms, b_ok = ds.batched(16, max(1, args.steps // 2), args.trials)
    b_best = min(b_ms, key=b_ms.get)
    out["decode_step_M16"] = {
        "workload": "the same 112-projection decode step for a batch of 16 tokens (grouped "
                    "launches; down's 16 x 8960 activations split over K ranges that meet "
                    "through atomics in the workspace)",
        "ms_per_step": {w: round(v, 5) for w, v in b_ms.items()}, "best": b_best,
        "tokens_per_s": round(16e3 / b_ms[b_best], 1),
        "weight_gb_per_s": round(ds.w_bytes / (b_ms[b_best] * 1e-3) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * ds.w_bytes / (b_ms[b_best] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "parity_ok": b_ok}
    log("decode step, M=16: " + ", ".join(
        f"{w} {v * 1e3:.1f} us ({ds.w_bytes / (v * 1e-3) / 1e9:.0f} GB/s of weights)"
        for w, v in b_ms.items()) + f"; parity {b_ok}")


CHAIN_FILE = os.path.join(ROOT, "profiles", "decode_chain_kernel_times.json")


def chain_kernel_times():
    """Sum of the profiler's kernel durations per chain step, per chain variant, from
    the committed kernel trace (None where the decode sources changed since)."""
    t = _traffic_file(CHAIN_FILE, DECODE_SOURCES)
    return None if t is None else t.get("chains")


def decode_chain_report(ds, med, ok):
    """The decode step as the dependent chain of single calls: (i) graph-replayed
    step time, (ii) the sum of the profiler's kernel times per step (committed
    trace), beside the grouped launch (iii) that the headline times."""
    kt = chain_kernel_times() or {}
    out = {"workload": "the 112 projections of one decode step (M=1) as single calls one "
                       "after another in decoder order (per layer qkv, o, gate_up, down), "
                       "every launch waiting for the one before; two steps per HIP graph "
                       "replay, the weight sets alternating",
           "parity_ok": ok}
    for name, key, launches in (("fused", "chain_fused_graph", 112),
                                ("two_launch", "chain_two_launch_graph", 224)):
        ms = med[key]
        gbs = ds.w_bytes / (ms * 1e-3) / 1e9
        row = {"launches_per_step": launches,
               "i_graph_ms_per_step": round(ms, 5),
               "i_tokens_per_s": round(1e3 / ms, 1),
               "i_weight_gb_per_s": round(gbs, 1),
               "i_pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        k = kt.get(name)
        if k:
            kus = k["kernel_us_per_step"]
            row["ii_kernel_time_sum_us_per_step"] = kus
            row["ii_weight_gb_per_s"] = round(ds.w_bytes / (kus * 1e-6) / 1e9, 1)
            row["ii_pct_of_hbm_peak"] = round(100 * ds.w_bytes / (kus * 1e-6) / 1e9 /
                                              HBM_PEAK_GBS, 2)
        else:
            row["ii_kernel_time_sum_us_per_step"] = None
        out[name] = row
    g = min(med["fused_eager"], med["two_launch_eager"], med["fused_graph"],
            med["two_launch_graph"])
    out["iii_grouped_ms_per_step"] = round(g, 5)
    return out


def run_chain_for_trace(torch, ds, replays: int):
    """The two decode chains alone, each graph replayed `replays` times (two steps
    per replay), for a kernel-trace pass: the per-step sum of kernel durations is
    then the trace's total for each chain's kernels over 2 * replays steps."""
    for fused in (True, False):
        g = capture_graph(torch, lambda: (ds.chain(0, fused), ds.chain(1, fused)))
        torch.cuda.synchronize()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        del g
        log(f"chain {'fused' if fused else 'two_launch'}: {replays} replays done")
    print(json.dumps({"chain_replays": replays, "steps_per_replay": 2,
                      "capture_steps_per_chain": 2}), flush=True)


def platform_versions(torch):
    """ROCm and HIP versions of the machine the numbers come from."""
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"rocm": rocm, "torch_hip": getattr(torch.version, "hip", None),
            "torch": torch.__version__, "device": props.name,
            "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count}


# --------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--layers", type=int, default=synth.N_LAYERS)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-singles", action="store_true")
    ap.add_argument("--no-ternarize", action="store_true")
    ap.add_argument("--no-i8s", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=6.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--batched", action="store_true",
                    help="also time the decode step for a batch of 16 tokens (off by default: "
                         "it runs the headline's kernel at another shape, which would mix into "
                         "that kernel's profiler averages)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the matrix-core issue-rate and streaming-read measurements")
    ap.add_argument("--remainder-counters", type=int, default=0, metavar="R",
                    help="only launch each remainder-sweep point R times eagerly (for a "
                         "profiler counter pass) and print the point order")
    ap.add_argument("--chain-only", action="store_true",
                    help="only replay the decode chain graphs (fused, then two-launch), "
                         "--steps replays each, for a kernel-trace pass of the profiler")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (5 times), to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    ap.add_argument("--clock-under-load", type=float, default=0.0, metavar="SECONDS",
                    help="only run the long-prefill stack's grouped GEMM launch back to back "
                         "for SECONDS (random int8 operands) and read the shader clock with "
                         "rocm-smi meanwhile")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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

    # torch before the library: libbt.so binds to the HIP runtime torch loads
    import torch

    if args.clock_under_load > 0:
        import ternary_weight_decoder_bt_amd as bt
        print(json.dumps(clock_under_load(torch, bt, args.clock_under_load)), flush=True)
        return

    packed_prefill = None
    if not args.no_prefill and not args.remainder_counters and not args.chain_only:
        t0 = time.time()
        packed_prefill = pack_long_prefill_weights(args.layers)
        log(f"long-prefill weights drawn and packed on the host in {time.time() - t0:.1f}s")

    import ternary_weight_decoder_bt_amd as bt
    bt.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.remainder_counters > 0:
        run_remainder_for_counters(torch, bt, dev, args.remainder_counters)
        return

    # ---- decode step (headline)
    ds = DecodeStep(torch, bt, dev, args.layers)
    if args.chain_only:
        run_chain_for_trace(torch, ds, args.steps)
        return
    check_idx = [0, 1, 2, 3, len(ds.items) - 1]
    ds.clear_outputs()
    ds.step_two_launch(0)
    torch.cuda.synchronize()
    two_launch_ok = ds.parity(check_idx)
    ds.clear_outputs()
    ds.step(0)
    torch.cuda.synchronize()
    decode_ok = ds.parity(check_idx) and two_launch_ok
    log(f"decode parity on sampled projections: fused {decode_ok}, two-launch {two_launch_ok}")

    def time_steps(step_fn, steps):
        """Step time: `steps` steps between two events, nothing recorded in between."""
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            step_fn(i)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    for i in range(args.warmup):
        ds.step(i)
        ds.step_two_launch(i)
    torch.cuda.synchronize()
    # HIP graphs of two consecutive steps (one per weight set): a replay runs
    # them with no host launch cost in between.
    g_fused = capture_graph(torch, lambda: (ds.step(0), ds.step(1)))
    g_two = capture_graph(torch, lambda: (ds.step_two_launch(0), ds.step_two_launch(1)))
    # the dependent chain: 112 single calls (or 224 launches) per step, in order
    g_chain_f = capture_graph(torch, lambda: (ds.chain(0, True), ds.chain(1, True)))
    g_chain_t = capture_graph(torch, lambda: (ds.chain(0, False), ds.chain(1, False)))
    graph_ok = True
    for g in (g_fused, g_two):
        ds.clear_outputs()
        g.replay()
        torch.cuda.synchronize()
        graph_ok = graph_ok and ds.parity(check_idx)
    decode_ok = decode_ok and graph_ok
    log(f"decode parity after graph replays: {graph_ok}")
    chain_ok = True
    for g in (g_chain_f, g_chain_t):
        ds.clear_outputs()
        g.replay()
        torch.cuda.synchronize()
        chain_ok = chain_ok and ds.parity(check_idx)
    log(f"decode chain parity after graph replays: {chain_ok}")
    # Timed trials: every variant in turn, repeated; the median of each is kept
    # (interleaving spreads clock and thermal drift over all variants alike).
    runs = {
        "fused_eager": (lambda i: ds.step(i), 1),
        "two_launch_eager": (lambda i: ds.step_two_launch(i), 1),
        "fused_graph": (lambda i: g_fused.replay(), 2),
        "two_launch_graph": (lambda i: g_two.replay(), 2),
        "gemv_fused_b2b": (lambda i: ds.fplans[i & 1].launch(), 1),
        "gemv_two_launch_b2b": (lambda i: ds.mplans[i & 1].launch(), 1),
    }
    # the dependent chains are timed in trials of their own, after the grouped
    # variants: interleaved with them, their long stretches of small latency-bound
    # launches left the next grouped variant measured 5-10% slow
    chain_runs = {
        "chain_fused_graph": (lambda i: g_chain_f.replay(), 2),
        "chain_two_launch_graph": (lambda i: g_chain_t.replay(), 2),
    }
    for _ in range(args.warmup):
        for fn, _per in list(runs.values()) + list(chain_runs.values()):
            fn(0)
    samples = {k: [] for k in list(runs) + list(chain_runs)}
    t_wall = time.perf_counter()
    for group in (runs, chain_runs):
        for _ in range(args.trials):
            for k, (fn, per) in group.items():
                # each variant's own untimed warm-up steps right before its timed ones
                for i in range(max(1, args.warmup // per)):
                    fn(i)
                samples[k].append(time_steps(fn, max(1, args.steps // per)) / per)
    t_wall = time.perf_counter() - t_wall
    med = {k: float(np.median(v)) for k, v in samples.items()}
    paths = {}
    for name, alg, kern, work in (
            ("fused", ds.alg_bytes, "gemv_grouped_kernel<true>",
             "one launch per step: quantization fused into the grouped GEMV"),
            ("two_launch", ds.alg_bytes_gemv, "gemv_grouped_kernel<false>",
             "two launches per step: grouped quantize, then grouped GEMV")):
        for mode in ("eager", "graph"):
            paths[f"{name}_{mode}"] = {
                "ms_per_step": med[f"{name}_{mode}"], "kernel_ms": [med[f"gemv_{name}_b2b"]],
                "alg": alg, "kernel": kern,
                "workload": work + ("; steps replayed from a HIP graph" if mode == "graph"
                                    else "; launched eagerly")}
    for k, v in med.items():
        log(f"decode [{k}]: {v * 1e3:.1f} us (median of {args.trials}; all: "
            f"{', '.join(f'{x * 1e3:.1f}' for x in samples[k])})")
    spread = {k: {"p10": round(float(np.percentile(v, 10)), 5),
                  "p50": round(float(np.median(v)), 5),
                  "p90": round(float(np.percentile(v, 90)), 5),
                  "trials_ms": [round(x, 5) for x in v]} for k, v in samples.items()}
    head_name = min(paths, key=lambda k: paths[k]["ms_per_step"])
    head = paths[head_name]
    ms_step = head["ms_per_step"]
    kern_avg_ms = float(np.mean(head["kernel_ms"]))
    value = ds.w_bytes / (ms_step * 1e-3) / 1e9
    achieved = head["alg"] / (kern_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(head["kernel"])
    log(f"headline path: {head_name}; timed region wall {t_wall:.2f}s")

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
                               "down 8960->1536 (" + head["workload"] + "); the 112 "
                               "projections of the synthetic step are independent and "
                               "overlap in the grouped launch (decode_chain.iii); a dependent "
                               "decoder runs them as the chain decode_chain.i",
                   "layers": args.layers, "M": 1, "weight_bytes_per_step": ds.w_bytes,
                   "weight_sets_alternating": 2, "path": head_name},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(1e3 / ms_step, 1),
        "tokens_per_s_basis": "grouped launch: the projections overlap (an upper bound for a "
                              "decoder, whose projections depend on one another)",
        "tokens_per_s_dependent_chain": round(1e3 / med["chain_fused_graph"], 1),
        "parity_ok": decode_ok,
        "roofline": {"bound": "hbm", "kernel": head["kernel"],
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": head["alg"],
                     "avg_launch_ms": round(kern_avg_ms, 5)},
        "decode_paths_ms_per_step": {k: round(v["ms_per_step"], 5) for k, v in paths.items()},
        "decode_trials_ms": spread,
        "decode_chain": decode_chain_report(ds, med, chain_ok),
        "gemv_kernel_ms_back_to_back": {"gemv_grouped_kernel<true>": round(med["gemv_fused_b2b"], 5),
                                        "gemv_grouped_kernel<false>":
                                            round(med["gemv_two_launch_b2b"], 5)},
        "timing": f"median of {args.trials} interleaved trials of {args.steps} steps per variant "
                  "(p10 / p90 of the trials in decode_trials_ms)",
        "platform": platform_versions(torch),
    }
    # ---- the same step for a batch of 16 tokens (batched decode)
    if args.batched:
        run_batched_decode(ds, out, args)

    # ---- the one-time device repack, timed on its own (not part of a step)
    rp = ds.time_repack()
    rp_bytes = 2 * ds.w_bytes   # read canonical + write tile layout (same size at these shapes)
    rp_ms = rp["grouped"]
    for k, v in rp.items():
        log(f"repack [{k}]: {v * 1e3:.1f} us for the stack ({rp_bytes / (v * 1e-3) / 1e9:.0f} GB/s)")
    out["repack"] = {
        "workload": "one-time device repack of the decode stack's 112 weight tensors "
                    "(canonical 2-bit layout -> tile layout) in one grouped launch",
        "ms_per_stack": round(rp_ms, 4), "bytes_per_stack": rp_bytes,
        "gb_per_s": round(rp_bytes / (rp_ms * 1e-3) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * rp_bytes / (rp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "ms_per_stack_one_launch_per_tensor_graph": round(rp["per_tensor_graph"], 4)}
    del ds
    torch.cuda.empty_cache()

    # A secondary leg that raises is recorded under "errors" and the rest still
    # runs, so the headline line is always printed.
    def guarded(name, fn):
        try:
            return fn()
        except Exception as e:  # noqa: BLE001
            log(f"{name} failed: {e!r}")
            out.setdefault("errors", {})[name] = repr(e)
            return None

    # ---- offline ternarization of the stack (one-time, like the repack)
    if not args.no_ternarize:
        out["ternarize"] = guarded("ternarize",
                                   lambda: run_ternarize_stack(torch, bt, dev, args.layers))

    # ---- single-projection calls (one GEMV, remainder sweep, one-layer prefill)
    if not args.no_singles:
        out["single_projections"] = guarded("single_projections",
                                            lambda: run_single_projections(torch, bt, dev))

    # ---- long prefill (secondary)
    def long_prefill_leg(packed):
        lp = LongPrefill(torch, bt, dev, args.layers, 4096, packed)
        packed.clear()
        try:
            return long_prefill_report(lp)
        finally:
            del lp
            torch.cuda.empty_cache()

    def long_prefill_report(lp):
        lp.step()
        torch.cuda.synchronize()
        pf_ok = lp.parity_sampled()
        # the whole stack (112 quantize + 112 GEMM launches) as one HIP graph
        g_stack = capture_graph(torch, lp.step)
        g_gemms = capture_graph(torch, lp.gemms)
        for p in lp.probs:
            p["y"].fill_(float("nan"))
        g_stack.replay()
        torch.cuda.synchronize()
        pf_ok = pf_ok and lp.parity_sampled()

        def replay_trials(gr):
            """Each of `prefill_steps` replays between its own two events (ms), after
            two untimed replays."""
            for _ in range(2):
                gr.replay()
            ts = []
            for _ in range(args.prefill_steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                a.record()
                gr.replay()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return ts

        def pcts(ts):
            return {"p10": round(float(np.percentile(ts, 10)), 4),
                    "p50": round(float(np.percentile(ts, 50)), 4),
                    "p90": round(float(np.percentile(ts, 90)), 4),
                    "trials_ms": [round(t_, 4) for t_ in ts]}

        trials = {"per_projection_stack": replay_trials(g_stack)}
        ms = float(np.median(trials["per_projection_stack"]))
        # GEMM-only time: the stack's GEMMs back to back (no quantize between)
        trials["per_projection_gemms"] = replay_trials(g_gemms)
        gemm_ms = float(np.median(trials["per_projection_gemms"]))
        tops = lp.ops / (ms * 1e-3) / 1e12
        gemm_tops = lp.ops / (gemm_ms * 1e-3) / 1e12
        # the grouped stack: one quantization launch, one GEMM launch
        lp.build_grouped()
        g_gstack = capture_graph(torch, lp.step_grouped)
        g_ggemm = capture_graph(torch, lp.ggplan.launch)
        for g_ in lp.gitems:
            g_["y"].fill_(float("nan"))
        g_gstack.replay()
        torch.cuda.synchronize()
        grouped_ok = lp.grouped_matches()
        times = {}
        for name, gr in (("stack", g_gstack), ("gemm", g_ggemm), ("per_projection_stack", g_stack)):
            trials["grouped_" + name if name != "per_projection_stack" else
                   "per_projection_stack_same_trial"] = ts_ = replay_trials(gr)
            times[name] = float(np.median(ts_))
        g_ms, gg_ms = times["stack"], times["gemm"]
        log(f"prefill grouped: {g_ms:.3f} ms/stack ({lp.ops / (g_ms * 1e-3) / 1e12:.0f} TOPS), "
            f"GEMM launch {gg_ms:.3f} ms ({lp.ops / (gg_ms * 1e-3) / 1e12:.0f} TOPS); "
            f"matches per-projection: {grouped_ok}")
        del g_gstack, g_ggemm
        shapes = lp.time_shapes()
        prologues = lp.time_activation_prologues()
        epilogues = lp.time_epilogues()
        for k_, (ms_, tops_) in epilogues.items():
            log(f"gemm {k_}: {ms_ * 1e3:.1f} us ({tops_:.0f} TOPS)")
        for k_, (ms_, gbs) in prologues.items():
            log(f"{k_}: {ms_ * 1e3:.1f} us ({gbs:.0f} GB/s, {100 * gbs / HBM_PEAK_GBS:.1f}% of HBM)")
        log(f"prefill: {ms:.3f} ms/stack ({tops:.0f} TOPS), GEMMs {gemm_ms:.3f} ms ({gemm_tops:.0f} TOPS)")
        return {
            "workload": "long prefill, M=4096 tokens x 28 layers x 4 projections (quantize + GEMM "
                        "each), replayed from a HIP graph",
            "int8_ops_per_stack": lp.ops, "ms_per_stack": round(ms, 4),
            "tops": round(tops, 2), "gemm_only_tops": round(gemm_tops, 2),
            "pct_of_int8_peak": round(100 * tops / I8_PEAK_TOPS, 2),
            "gemm_only_pct_of_int8_peak": round(100 * gemm_tops / I8_PEAK_TOPS, 2),
            "parity_sampled_ok": pf_ok,
            "parity_sampled": "q of the first and last projection in full; y on 4 rows and "
                              "4 columns of each (every output of all 112 projections is "
                              "compared by tests/test_gpu_long_prefill_full.py)",
            "steps": args.prefill_steps,
            "trials": {k: pcts(v) for k, v in trials.items()},
            "timing": "each figure is the median over `steps` graph replays, each between its "
                      "own two events, after two untimed replays",
            "grouped": {
                "workload": "the same stack as one grouped quantization launch over the 112 "
                            "inputs and one grouped GEMM launch over the 112 projections (the "
                            "projections are independent here, as in the grouped decode step)",
                "ms_per_stack": round(g_ms, 4), "tops": round(lp.ops / (g_ms * 1e-3) / 1e12, 2),
                "pct_of_int8_peak": round(100 * lp.ops / (g_ms * 1e-3) / 1e12 / I8_PEAK_TOPS, 2),
                "gemm_ms": round(gg_ms, 4),
                "gemm_tops": round(lp.ops / (gg_ms * 1e-3) / 1e12, 2),
                "gemm_pct_of_int8_peak": round(100 * lp.ops / (gg_ms * 1e-3) / 1e12 /
                                               I8_PEAK_TOPS, 2),
                "matches_per_projection_bitwise": grouped_ok,
                "per_projection_ms_same_trial": round(times["per_projection_stack"], 4)},
            "gemm_tops_per_shape": {k: round(v[1], 1) for k, v in shapes.items()},
            "gemm_us_per_shape": {k: round(v[0] * 1e3, 2) for k, v in shapes.items()},
            "gemm_epilogues": {k: {"us": round(v[0] * 1e3, 2), "tops": round(v[1], 1)}
                               for k, v in epilogues.items()},
            "activation_prologues": {
                k: {"us": round(v[0] * 1e3, 2), "gb_per_s": round(v[1], 1),
                    "pct_of_hbm_peak": round(100 * v[1] / HBM_PEAK_GBS, 2)}
                for k, v in prologues.items()},
            "roofline": {"bound": "mfma",
                         "kernel": "gemm_persistent_grouped_kernel (the stack's 112 GEMMs in "
                                   "one launch)",
                         "achieved": round(lp.ops / (gg_ms * 1e-3) / 1e12, 2),
                         "peak": I8_PEAK_TOPS, "unit": "TFLOP/s",
                         "frac": round(lp.ops / (gg_ms * 1e-3) / 1e12 / I8_PEAK_TOPS, 4),
                         "traffic": measured_gemm_traffic("grouped"),
                         "traffic_unit": "HBM bytes per grouped GEMM launch (the whole stack)",
                         "algorithmic_bytes_per_launch": lp.alg_bytes,
                         "per_projection": {
                             "kernels": "gemm_persistent_kernel (gate_up) + gemm_kernel (qkv, "
                                        "o, down), 112 launches",
                             "achieved": round(gemm_tops, 2),
                             "frac": round(gemm_tops / I8_PEAK_TOPS, 4),
                             "traffic": measured_gemm_traffic("per_projection")}},
        }

    if not args.no_prefill:
        out["prefill"] = guarded("prefill", lambda: long_prefill_leg(packed_prefill))
        del packed_prefill

    # ---- I8_S (the tokenizer's INT8 GEMMs), secondary
    if not args.no_i8s:
        out["i8s"] = guarded("i8s", lambda: run_i8s_tokenizer_ffn(torch, bt, dev))

    if not args.no_ceilings:
        out["ceilings"] = c = guarded("ceilings", lambda: run_ceilings(torch, dev))
        if c:
            log(f"ceilings: int8 MFMA {c['int8_peak_tops_measured']} TOPS measured "
                f"({c['int8_peak_tops_derived_at_2p4ghz']} at 2.4 GHz), streaming read "
                f"{c['stream_read_peak_gb_per_s']} GB/s")

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = guarded("cpu_baseline", lambda: cpu_baseline(args.cpu_seconds))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
