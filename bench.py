#!/usr/bin/env python3
"""Benchmark of the Prox sparse SwiGLU FFN decode step on one MI355X.

Metric: microseconds per FFN layer, plus achieved HBM GB/s and the fraction of
the 8 TB/s roofline on the bytes the method must move, at 70% intermediate
sparsity and 50% input keep, batch 1, on a Qwen3-8B-shaped layer
(d_model 4096, d_ff 12288, bf16 weights, fp32 accumulation).

Method of measurement
  * 8 independent seeded layers (2.8 GB of packed weights) are rotated so the
    256 MB Infinity Cache cannot hold the working set; each step decodes one
    seeded Laplace token through one layer (prox_ffn_decode: three kernels).
  * The headline number times exactly K steps replayed from HIP graphs (the
    per-step GPU work is tens of microseconds, shorter than eager host launch
    overhead); the eager rate is reported beside it.
  * Each kernel is also replayed alone over the same steps (HIP events on the
    stream the kernels run on); the dominant kernel's algorithmic bytes over
    its mean duration is the roofline figure.  The opt-in fused Stage-2
    kernel (a cooperative launch) is timed beside them unless --no-fused
    (kernel-trace runs use it: rocprofv3 loses its trace output after
    cooperative launches).
  * Required bytes use the actual k_x and k_s of each timed step, averaged
    over exactly the K timed steps:
    k_x*d_ff (INT4 up+gate rows) + 8*k_x (scales) + 3*k_s*d_model*2 (kept bf16
    rows of W_up^T, W_gate^T, W_down) + 2*d_model (x) + 4*d_model (y) + 4*k_s.
  * Dense comparators on the same rotation: torch bf16 (one fused up/gate
    GEMV, SiLU, product, down GEMV) and this library's Stage-2 kernels with
    every channel kept.
  * Other configurations (the `configs` block): the 36-layer Qwen3-8B-shaped
    stack swept over intermediate sparsity 0.5 / 0.6 / 0.7, and the
    Qwen3-32B-shaped layer, each with its own roofline and dense comparators.
  * CPU baseline: the plain NumPy oracle on the host cores (median over a
    bounded sample of layer 0's tokens; single-thread runs of one 8B layer
    and of the tiny layer), plus the agreement of the GPU's masks and y with
    the oracle's on those tokens.
  * Computation budget (the pages' budget section): alpha = Stage 1 over
    every input / one dense bf16 projection, both timed here; the library's
    allocator (prox_budget_s2) gives s2 for a target effective sparsity at
    input sparsity 0.7, the layers are recalibrated and the decode is timed
    at each such operating point (and at the pages' alpha = 1/3).

Prints one JSON line on stdout; progress goes to stderr.  Other modes:
  --pmc-copy-mib N          device copies of N MiB (counter scale reference)
  --pmc-run WORKLOAD        one eager pass of the decode over a workload's
                            rotation, for rocprofv3 --pmc; writes the
                            algorithmic bytes of those launches to --pmc-meta
  --summarize-pmc DIR       turns rocprofv3 FETCH_SIZE / WRITE_SIZE runs under
                            DIR into profiles/traffic.json records and a
                            markdown table
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per FFN layer + achieved HBM GB/s (% roofline) at 70% sparsity, batch 1"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# Decode kernels: the sources that define each one, and the substrings of the
# kernel names rocprofv3 reports for it (a step of the grouped down stage is
# two kernels, whose counters add up).
KERNELS = {
    "stage1_proxy": (("stage1.hip",), ("stage1_kernel<prox::Bf16Tag, false, true>",)),
    "stage2_fused": (("stage2_fused.hip", "stage2_common.h"), ("stage2_fused_kernel<prox::Bf16Tag>",)),
    "stage2_upgate": (("stage2_upgate.hip", "stage2_common.h"), ("upgate_kernel<prox::Bf16Tag, true, true>",)),
    "stage2_down": (("stage2_down.hip", "stage2_common.h"), ("down_kernel<prox::Bf16Tag, true, true>",)),
    "stage1_proxy_batch": (("stage1_qt.hip", "stage1_mfma.h"), ("stage1_qt_kernel<prox::Bf16Tag, false, 1>",)),
    "stage2_upgate_batch": (("stage2_batch.hip",), ("upgate_batch_kernel",)),
    "stage2_down_batch": (("stage2_batch.hip",), ("down_batch_kernel", "down_reduce_kernel")),
}
STAGE_NAMES = ["stage1_proxy", "stage2_upgate", "stage2_down"]  # the decode step's kernels


def kernel_source_hash(kernel: str) -> str:
    """sha256 over the sources that define a kernel's code."""
    csrc = os.path.join(ROOT, "free_ffn_activation_amd", "csrc")
    h = hashlib.sha256()
    for name in (*KERNELS[kernel][0], "prox_device.h", "prox_internal.h"):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_key(workload: str, d: int, f: int, keep_x: float, sparsity_s: float, batch: int) -> dict:
    return {"workload": workload, "d_model": int(d), "d_ff": int(f), "keep_x": round(float(keep_x), 4),
            "sparsity_s": round(float(sparsity_s), 4), "batch": int(batch)}


def measured_traffic(kernel: str, key: dict, algorithmic_bytes: float):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record of this kernel on this workload (shape, keep fractions, batch), or
    None when there is none or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            recs = json.load(fh).get("records", [])
    except (OSError, ValueError):
        return None
    sha = kernel_source_hash(kernel)
    for rec in recs:
        if rec.get("kernel") == kernel and all(rec.get(k) == v for k, v in key.items()):
            if rec.get("source_sha256") != sha:
                return None
            return {"bytes_per_launch": rec["hbm_bytes_per_launch"],
                    "fetch_bytes": rec["fetch_bytes_per_launch"], "write_bytes": rec["write_bytes_per_launch"],
                    "vs_algorithmic": round(rec["hbm_bytes_per_launch"] / algorithmic_bytes, 3)}
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1280)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="qwen3_8b", choices=["qwen3_8b", "qwen3_32b"],
                    help="configuration of the headline line")
    ap.add_argument("--layers", type=int, default=None, help="layer instances rotated")
    ap.add_argument("--sparsity", type=float, default=0.7)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-fused", action="store_true",
                    help="leave out the opt-in fused Stage-2 timings (kernel-trace runs: rocprofv3 loses its "
                         "trace output after the kernel's cooperative launches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-budget", action="store_true",
                    help="skip the computation-budget, calibration, 16-bit proxy and GeGLU sections")
    ap.add_argument("--no-batch", action="store_true",
                    help="skip the batch-8 decode (grouped kernels vs per-token kernels vs dense)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 36-layer sparsity sweep and the Qwen3-32B-shaped layer")
    ap.add_argument("--config-steps", type=int, default=256, help="timed steps of the 32B configuration")
    ap.add_argument("--records", default=None, help="write one JSON record per (config, layer, token) here")
    ap.add_argument("--pmc-copy-mib", type=int, default=0,
                    help="only run device copies of this many MiB (counter scale reference)")
    ap.add_argument("--pmc-run", default=None, choices=["qwen3_8b", "qwen3_32b"],
                    help="only run one eager decode pass over this workload's rotation (counter runs)")
    ap.add_argument("--pmc-batch", type=int, default=1, help="tokens per decode call in --pmc-run (1 or 8)")
    ap.add_argument("--pmc-meta", default=None, help="--pmc-run: write the launches' algorithmic bytes here")
    ap.add_argument("--summarize-pmc", default=None, help="directory of rocprofv3 counter runs to summarise")
    return ap.parse_args()


# ============================================================================ GPU-side helpers
class Rotation:
    """n_layers seeded layers of one configuration, packed and resident, with
    n_tok decode tokens each; step s decodes token (s // n_layers) % n_tok of
    layer s % n_layers, so consecutive steps read different layers."""

    def __init__(self, cfg, n_layers: int, n_tok: int = 16, first_layer: int = 0):
        import numpy as np
        import torch
        from concurrent.futures import ThreadPoolExecutor

        import synth
        from free_ffn_activation_amd import prox
        from free_ffn_activation_amd.upload import pack_layer, to_device

        self.cfg, self.n_layers, self.n_tok = cfg, n_layers, n_tok
        self.d, self.f = cfg.d_model, cfg.d_ff
        dev = torch.device("cuda:0")
        self.layers, self.x_cal = [], []
        self.x_all = torch.empty(n_layers, n_tok, self.d, dtype=torch.int16 if cfg.dtype == "bf16" else torch.float32,
                                 device=dev)
        self.host0 = None
        t0 = time.time()
        chunk = 8
        with ThreadPoolExecutor(8) as ex:
            for c0 in range(0, n_layers, chunk):
                idx = list(range(c0, min(n_layers, c0 + chunk)))
                hosts = list(ex.map(lambda i: synth.make_layer(cfg, first_layer + i, n_dec=n_tok), idx))
                for i, hl in zip(idx, hosts):
                    self.layers.append(pack_layer(hl))
                    self.x_cal.append(to_device(hl.x_cal, cfg.dtype))
                    self.x_all[i].copy_(to_device(hl.x_dec, cfg.dtype))
                    if i == 0:
                        self.host0 = hl
                del hosts
        torch.cuda.synchronize()
        log(f"{cfg.name}: {n_layers} layers generated and packed in {time.time() - t0:.1f}s "
            f"({sum(L.nbytes for L in self.layers) / 1e9:.2f} GB resident)")
        self.xs = [[self.x_all[l, t:t + 1] for t in range(n_tok)] for l in range(n_layers)]
        self.steps_per_round = n_layers * n_tok
        self.sched = [(s % n_layers, (s // n_layers) % n_tok) for s in range(self.steps_per_round)]
        self.cal_ws = torch.empty(prox.prox_calibrate_workspace_size(self.d, self.f, cfg.n_cal), dtype=torch.uint8,
                                  device=dev)
        self.np = np

    def calibrate(self, keep_x: float, sparsity_s: float, layers=None):
        from free_ffn_activation_amd import prox
        layers = layers or self.layers
        return [prox.prox_calibrate(layers[l], self.x_cal[l], keep_x, sparsity_s, self.cal_ws)
                for l in range(self.n_layers)]

    def at(self, s):
        return self.sched[s % self.steps_per_round]

    def tmean(self, a, K: int) -> float:
        """Mean of a per-(layer, token) array over exactly the steps 0..K-1."""
        return float(self.np.mean([a[self.at(s)] for s in range(K)]))

    def free(self):
        import torch
        self.layers.clear()
        self.x_cal.clear()
        del self.x_all, self.xs, self.cal_ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


class Outs:
    """Output buffers of one decode call of `b` tokens."""

    def __init__(self, d, f, b=1):
        import torch
        from free_ffn_activation_amd import prox
        self.y = torch.empty(b, d, dtype=torch.float32, device="cuda")
        self.mi = torch.empty(b, f, dtype=torch.int32, device="cuda")
        self.mc = torch.empty(b, dtype=torch.int32, device="cuda")
        self.ic = torch.empty(b, dtype=torch.int32, device="cuda")
        self.ws = prox.new_workspace(d, f, b)


# Device cycles of the spin kernel queued ahead of a timed region (about
# 0.4 ms): the start event then executes after the host has queued the
# replays, so the host's submission latency of the first graph (tens of us)
# is not counted as GPU time of the K steps.
LEAD_CYCLES = 1_000_000
# Untimed replays of the timed graphs right before the timed region (the
# warm-up steps): measured on the 8B layer, a 20-step window timed right
# after setup read 33.6 us per step and 32.5 us after other GPU work (a
# 20-step bench run: 33.7 us without these replays, 33.0 us after 256; with
# the current kernels three 20-step runs read 30.57 / 30.72 / 30.50 us after
# 256 and 30.36 / 30.54 / 30.43 us after 1024).  The warm replays end on the
# window's last steps, whose data the first timed steps do not read, so no
# timed step finds its weights in a cache because of them.
WARM_STEPS = 1024


def time_graph(fn, steps_per_round: int, K: int, label: str, graph: bool = True) -> float:
    """Exactly K steps (fn(0) .. fn(K-1)) replayed from HIP graphs (whole
    rotations of steps_per_round steps, then a graph of the first
    K mod steps_per_round), after at least WARM_STEPS untimed steps replayed
    from the same graphs, bracketed by HIP events on the current stream,
    behind a short spin kernel so that the events time the GPU's execution of
    the K steps, not the host's submission of the first graph.  Returns
    microseconds per step."""
    import torch
    if not graph:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            fn(s)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / K * 1e6
        log(f"{label}: {us:.2f} us/step over {K} eager steps")
        return us
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for s in range(min(K, steps_per_round)):  # warm the capture stream
            fn(s)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(n):
                fn(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        return g

    full, tail = divmod(K, steps_per_round)
    g_full = capture(steps_per_round) if full else None
    g_tail = capture(tail) if tail else None
    warm = g_full if g_full is not None else g_tail
    for _ in range(max(1, -(-WARM_STEPS // (steps_per_round if g_full is not None else tail)))):
        warm.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(LEAD_CYCLES)
    ev0.record()
    for _ in range(full):
        g_full.replay()
    if g_tail is not None:
        g_tail.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / K
    log(f"{label}: {us:.2f} us/step over {K} graph-replayed steps")
    del g_full, g_tail
    return us


def decode_counts(rot, taus, layers=None, out=None):
    """k_x and k_s of every (layer, token) under the thresholds taus."""
    import torch
    from free_ffn_activation_amd import prox
    np = rot.np
    layers = layers or rot.layers
    out = out or Outs(rot.d, rot.f)
    kx = np.zeros((rot.n_layers, rot.n_tok), np.int64)
    ks = np.zeros((rot.n_layers, rot.n_tok), np.int64)
    for l in range(rot.n_layers):
        for t in range(rot.n_tok):
            prox.prox_ffn_decode(layers[l], rot.xs[l][t], taus[l][0], taus[l][1], out.y, out.mi, out.mc, out.ic, out.ws)
            torch.cuda.synchronize()
            kx[l, t], ks[l, t] = int(out.ic.item()), int(out.mc.item())
    return kx, ks


def byte_model(kx, ks, d: int, f: int, w: int):
    """Algorithmic bytes per (layer, token): the whole step and each kernel."""
    ug = 2 * ks * d * w + d * w + f // 8 + 8 * ks
    dn = ks * d * w + 8 * ks + 4 * d
    return {"step": kx * f + 8 * kx + 3 * ks * d * w + d * w + 4 * d + 4 * ks,
            "stage1_proxy": kx * f + 8 * kx + d * w + f // 8,
            "stage2_upgate": ug, "stage2_down": dn, "stage2_fused": ug + dn}


def per_step_events(rot, fn, n: int):
    """Eager steps 0..n-1, a HIP event pair around each: microseconds per step."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for s in range(n):
        evs[s][0].record()
        fn(s)
        evs[s][1].record()
    torch.cuda.synchronize()
    return rot.np.array([a.elapsed_time(b) * 1e3 for a, b in evs])


def measure_decode(rot, taus, K: int, workload: str, keep_x: float, sparsity_s: float, args, kernels_alone=True,
                   dense=True, records=None):
    """The decode over the rotation: graph-timed K steps, eager rate and
    per-step distribution, each kernel alone, roofline of the dominant kernel,
    dense comparators.  Required and per-kernel bytes are averaged over
    exactly the K timed steps."""
    import torch
    from free_ffn_activation_amd import prox
    np = rot.np
    d, f, n = rot.d, rot.f, rot.n_layers
    w = 2 if rot.cfg.dtype == "bf16" else 4
    spr = rot.steps_per_round
    o = Outs(d, f)
    kx, ks = decode_counts(rot, taus, out=o)
    bm = byte_model(kx, ks, d, f, w)

    def step(s):
        l, t = rot.at(s)
        prox.prox_ffn_decode(rot.layers[l], rot.xs[l][t], taus[l][0], taus[l][1], o.y, o.mi, o.mc, o.ic, o.ws)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(s)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) / K * 1e6
    # per-step distribution over whole rotations (every (layer, token) at least once)
    n_ev = max(spr, min(K, 640))
    per = per_step_events(rot, step, n_ev)
    dist = {"median": round(float(np.median(per)), 3), "p10": round(float(np.percentile(per, 10)), 3),
            "p90": round(float(np.percentile(per, 90)), 3), "steps": int(n_ev),
            "timing": "eager, hipEvent pair per step"}
    us = time_graph(step, spr, K, f"{workload} decode (keep_x {keep_x}, s2 {sparsity_s})", graph=not args.no_graph)
    breq = rot.tmean(bm["step"], K)
    gbps = breq / (us * 1e-6) / 1e9
    res = {"us_per_layer": round(us, 3), "eager_us_per_layer": round(eager_us, 3), "step_us": dist,
           "timed_steps": K, "required_MB_per_layer": round(breq / 1e6, 3), "achieved_GBps": round(gbps, 1),
           "pct_hbm_roofline": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
           "mean_k_x": round(rot.tmean(kx, K), 1), "mean_k_s": round(rot.tmean(ks, K), 1)}
    if records is not None:
        per_lt = {}
        for s in range(n_ev):
            per_lt.setdefault(rot.at(s), []).append(float(per[s]))
        for (l, t), v in sorted(per_lt.items()):
            records.append({"config": workload, "keep_x": keep_x, "sparsity_s": sparsity_s, "layer": l, "token": t,
                            "k_x": int(kx[l, t]), "k_s": int(ks[l, t]), "us_eager_event": round(min(v), 3),
                            "required_bytes": int(bm["step"][l, t])})
    if kernels_alone:
        # each kernel alone over the same K steps: every schedule step owns a
        # workspace and outputs prepared by one full decode
        iso = [Outs(d, f) for _ in range(spr)]

        def staged(stages):
            def fn(s):
                l, t = rot.at(s)
                b = iso[s % spr]
                prox.prox_ffn_decode_stages(rot.layers[l], rot.xs[l][t], taus[l][0], taus[l][1], b.y, b.mi, b.mc,
                                            b.ic, b.ws, stages)
            return fn

        full = staged(7)
        for s in range(spr):
            full(s)
        torch.cuda.synchronize()
        # the step's three kernels, then the fused Stage-2 kernel (opt-in,
        # PROX_STAGE_FUSED_STAGE2) for comparison
        fused = prox.PROX_STAGE_FUSED_STAGE2
        runs = [("stage1_proxy", prox.PROX_STAGE_PROXY), ("stage2_upgate", prox.PROX_STAGE_UPGATE),
                ("stage2_down", prox.PROX_STAGE_DOWN)]
        if not args.no_fused:
            runs.append(("stage2_fused", prox.PROX_STAGE_UPGATE | prox.PROX_STAGE_DOWN | fused))
        k_us = {nm: time_graph(staged(b), spr, K, f"{workload} {nm} alone", graph=not args.no_graph)
                for nm, b in runs}
        if not args.no_graph and not args.no_fused:
            res["us_per_layer_fused_stage2"] = round(
                time_graph(staged(7 | fused), spr, K, f"{workload} decode, Stage 2 fused (opt-in)"), 3)
        del iso
        kb = {nm: rot.tmean(bm[nm], K) for nm, _ in runs}
        dom = max(STAGE_NAMES, key=lambda nm: k_us[nm])
        ach = kb[dom] / (k_us[dom] * 1e-6) / 1e9
        key = traffic_key(workload, d, f, keep_x, sparsity_s, 1)
        traffic = measured_traffic(dom, key, kb[dom])
        res["kernels"] = {nm: {"us": round(k_us[nm], 3), "algorithmic_MB": round(kb[nm] / 1e6, 3),
                               "GBps": round(kb[nm] / (k_us[nm] * 1e-6) / 1e9, 1)} for nm, _ in runs}
        res["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1),
                           "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                           "traffic": traffic["bytes_per_launch"] if traffic else None,
                           "traffic_detail": traffic, "algorithmic_bytes_per_launch": round(kb[dom]),
                           "traffic_key": key}
        log(f"{workload} kernels alone: " + ", ".join(f"{nm} {u:.2f}" for nm, u in k_us.items()))
    if dense and not args.no_dense and rot.cfg.dtype == "bf16":
        res["dense_us_per_layer"] = dense_comparators(rot, K, o, args)
    return res, kx, ks


def dense_comparators(rot, K, o, args):
    """torch bf16 dense SwiGLU (fused up/gate linear, SiLU, product, down
    matmul) and this library's Stage 2 with every channel kept, same rotation."""
    import torch
    from free_ffn_activation_amd import prox
    d, f = rot.d, rot.f
    wug = [L.w_upgate_t.view(torch.bfloat16).view(2 * f, d) for L in rot.layers]
    wdn = [L.w_down.view(torch.bfloat16).view(f, d) for L in rot.layers]
    yb = torch.empty(1, d, dtype=torch.bfloat16, device="cuda")

    def dense_torch(s):
        l, t = rot.at(s)
        ug = torch.nn.functional.linear(rot.xs[l][t].view(torch.bfloat16), wug[l])
        sv = ug[:, 0::2] * torch.nn.functional.silu(ug[:, 1::2])
        torch.matmul(sv, wdn[l], out=yb)

    all_j = torch.arange(f, dtype=torch.int32, device="cuda").view(1, f)
    all_c = torch.full((1,), f, dtype=torch.int32, device="cuda")

    def dense_own(s):
        l, t = rot.at(s)
        prox.prox_ffn_stage2(rot.layers[l], rot.xs[l][t], all_j, all_c, o.y, o.ws)

    out = {}
    for fn, label in ((dense_torch, "dense_torch_bf16"), (dense_own, "dense_own_stage2")):
        for s in range(8):
            fn(s)
        torch.cuda.synchronize()
        out[label] = round(time_graph(fn, rot.steps_per_round, K, label, graph=not args.no_graph), 3)
    return out


# ============================================================================ sections
def stack_sweep(args, records):
    """36 independent seeded Qwen3-8B-shaped layers, one decode token per layer
    per pass, rotated as a whole (12.7 GB resident); intermediate sparsity
    0.5 / 0.6 / 0.7 at input keep 0.5 (thresholds recalibrated per point)."""
    import synth
    cfg = synth.CONFIGS["qwen3_8b_stack"]
    rot = Rotation(cfg, 36, 16)
    K = rot.steps_per_round  # 576 steps: every layer 16 times
    points = []
    dense = None
    for s2 in (0.5, 0.6, 0.7):
        taus = rot.calibrate(cfg.keep_x, s2)
        res, _, _ = measure_decode(rot, taus, K, "qwen3_8b_stack36", cfg.keep_x, s2, args, kernels_alone=False,
                                   dense=False, records=records)
        res["us_per_stack"] = round(36 * res["us_per_layer"], 2)
        res["sparsity_s"] = s2
        points.append(res)
    if not args.no_dense:
        dense = dense_comparators(rot, K, Outs(rot.d, rot.f), args)
        dense = {k: {"us_per_layer": v, "us_per_stack": round(36 * v, 2)} for k, v in dense.items()}
    rot.free()
    return {"workload": "qwen3_8b_stack36", "d_model": cfg.d_model, "d_ff": cfg.d_ff, "layers": 36,
            "tokens_per_layer": 16, "keep_x": cfg.keep_x, "timed_steps_per_point": K, "points": points,
            "dense": dense}


def budget_section(rot, taus, alpha_parts, args):
    """The pages' computation budget: alpha measured here, s2 from the
    allocator for target effective sparsities at s1 = 0.7, decode timed at
    each point (and at the pages' alpha = 1/3)."""
    import torch
    from free_ffn_activation_amd import prox
    d, f = rot.d, rot.f
    K = max(1, args.steps)
    o = Outs(d, f)

    def s1_all_inputs(s):
        l, t = rot.at(s)
        prox.prox_ffn_decode_stages(rot.layers[l], rot.xs[l][t], 0.0, taus[l][1], o.y, o.mi, o.mc, o.ic, o.ws,
                                    prox.PROX_STAGE_PROXY)

    t_s1_all = time_graph(s1_all_inputs, rot.steps_per_round, K, "stage 1 over every input", graph=not args.no_graph)
    wug = [L.w_upgate_t.view(torch.bfloat16).view(2 * f, d) for L in rot.layers]

    def torch_two_projections(s):
        l, t = rot.at(s)
        torch.nn.functional.linear(rot.xs[l][t].view(torch.bfloat16), wug[l])

    all_j = torch.arange(f, dtype=torch.int32, device="cuda").view(1, f)
    all_c = torch.full((1,), f, dtype=torch.int32, device="cuda")

    def own_three_projections(s):
        l, t = rot.at(s)
        prox.prox_ffn_stage2(rot.layers[l], rot.xs[l][t], all_j, all_c, o.y, o.ws)

    t_proj_torch = time_graph(torch_two_projections, rot.steps_per_round, K, "torch bf16 up+gate projections",
                              graph=not args.no_graph) / 2
    t_proj_own = time_graph(own_three_projections, rot.steps_per_round, K, "own dense Stage 2 (3 projections)",
                            graph=not args.no_graph) / 3
    t_proj = min(t_proj_torch, t_proj_own)
    alpha = t_s1_all / t_proj
    alpha_parts.update(alpha=alpha, t_proj=t_proj)
    log(f"alpha = {t_s1_all:.2f} / {t_proj:.2f} = {alpha:.3f}")
    points = [("pages' alpha", 0.7, 0.7, 1.0 / 3.0)] + [("measured alpha", e, 0.7, alpha) for e in (0.5, 0.6, 0.7)]
    op_out = []
    for label, e_t, s1, a in points:
        try:
            s2 = prox.prox_budget_s2(e_t, s1, a)
        except prox.ProxError as exc:
            if exc.status != prox.PROX_ERR_UNSUPPORTED:
                raise
            op_out.append({"alpha_from": label, "e_target": e_t, "s1": s1, "alpha": round(a, 4),
                           "reachable": False, "reason": str(exc)})
            continue
        taus_op = rot.calibrate(1.0 - s1, s2)
        kx_o, ks_o = decode_counts(rot, taus_op, out=o)
        breq_o = byte_model(kx_o, ks_o, d, f, 2)["step"]

        def step_op(s, taus_op=taus_op):
            l, t = rot.at(s)
            prox.prox_ffn_decode(rot.layers[l], rot.xs[l][t], taus_op[l][0], taus_op[l][1], o.y, o.mi, o.mc, o.ic,
                                 o.ws)

        us_o = time_graph(step_op, rot.steps_per_round, K, f"decode at e={e_t} s1={s1} s2={s2:.4f} ({label})",
                          graph=not args.no_graph)
        mb = rot.tmean(breq_o, K)
        keep_x_run, keep_s_run = rot.tmean(kx_o, K) / d, rot.tmean(ks_o, K) / f
        op_out.append({"alpha_from": label, "e_target": e_t, "s1": s1, "s2": round(s2, 4),
                       "alpha": round(a, 4), "reachable": True, "us_per_layer": round(us_o, 3),
                       "required_MB": round(mb / 1e6, 3), "GBps": round(mb / (us_o * 1e-6) / 1e9, 1),
                       "pct_hbm_roofline": round(100.0 * mb / (us_o * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                       "runtime_keep_x": round(keep_x_run, 4), "runtime_keep_s": round(keep_s_run, 4),
                       "runtime_effective_sparsity": round(
                           prox.prox_budget_effective(1.0 - keep_x_run, 1.0 - keep_s_run, a), 4)})
    return {"alpha": round(alpha, 4), "t_stage1_all_inputs_us": round(t_s1_all, 3),
            "t_dense_projection_us": round(t_proj, 3), "t_dense_projection_torch_us": round(t_proj_torch, 3),
            "t_dense_projection_own_us": round(t_proj_own, 3), "operating_points": op_out}


def calibration_section(rot, alpha):
    """The pages calibrate with at most 200,000 samples and a 4,096-bin
    histogram per layer, in depth order, and report the runtime effective
    sparsity against each target.  Here the rotation's layers form a chain
    with a residual stream h (fp32): h_0 = x_0, h_{l+1} = h_l + y_l, and layer
    l+1 reads x_{l+1} = bf16(RMSNorm(h_{l+1})); for each target e at s1 = 0.7
    (s2 from the budget allocator with the measured alpha) every layer is
    calibrated on the chain's calibration tokens after the earlier layers ran
    sparse, then held-out tokens run through the chain and their keep
    fractions give the runtime effective sparsity."""
    import numpy as np
    import torch
    from free_ffn_activation_amd import prox
    d, f, n_layers, n_tok = rot.d, rot.f, rot.n_layers, rot.n_tok
    nb_h, ms_h = 4096, 200000
    n_cal = rot.x_cal[0].shape[0]
    hws = torch.empty(prox.prox_calibrate_hist_workspace_size(d, f, n_cal, ms_h, nb_h), dtype=torch.uint8,
                      device="cuda")
    co = Outs(d, f, n_cal)
    ho = Outs(d, f, n_tok)

    def rms_norm_bf16(h):  # fp32 residual stream -> bf16 bits of the normalised FFN input
        xn = h * torch.rsqrt(torch.mean(h * h, dim=-1, keepdim=True) + 1e-6)
        return xn.to(torch.bfloat16).view(torch.int16).contiguous()

    targets = []
    t_cal0 = time.perf_counter()
    for e_t in (0.4, 0.5, 0.6, 0.7):
        s1c = 0.7
        try:
            s2c = prox.prox_budget_s2(e_t, s1c, alpha)
        except prox.ProxError as exc:  # target out of reach at this alpha
            if exc.status != prox.PROX_ERR_UNSUPPORTED:
                raise
            targets.append({"e_target": e_t, "s1": s1c, "reachable": False, "reason": str(exc)})
            continue
        xc_chain = rot.x_cal[0].clone()
        hc = xc_chain.view(torch.bfloat16).float()
        thr = []
        for l in range(n_layers):
            tx, ts = prox.prox_calibrate_hist(rot.layers[l], xc_chain, 1.0 - s1c, s2c, hws, ms_h, nb_h)
            thr.append((tx, ts))
            prox.prox_ffn_decode(rot.layers[l], xc_chain, tx, ts, co.y, co.mi, co.mc, None, co.ws)
            hc = hc + co.y
            xc_chain = rms_norm_bf16(hc)
        xh = rot.x_all[0].clone()
        hh = xh.view(torch.bfloat16).float()
        kx_l, ks_l, e_l = [], [], []
        for l in range(n_layers):
            prox.prox_ffn_decode(rot.layers[l], xh, thr[l][0], thr[l][1], ho.y, ho.mi, ho.mc, ho.ic, ho.ws)
            torch.cuda.synchronize()
            kx_f = float(ho.ic.float().mean()) / d
            ks_f = float(ho.mc.float().mean()) / f
            kx_l.append(kx_f)
            ks_l.append(ks_f)
            e_l.append(prox.prox_budget_effective(1.0 - kx_f, 1.0 - ks_f, alpha))
            hh = hh + ho.y
            xh = rms_norm_bf16(hh)
        e_run = float(np.mean(e_l))
        targets.append({"e_target": e_t, "s1": s1c, "s2": round(s2c, 4), "reachable": True,
                        "runtime_keep_x_mean": round(float(np.mean(kx_l)), 4),
                        "runtime_keep_s_mean": round(float(np.mean(ks_l)), 4),
                        "runtime_effective_mean": round(e_run, 4),
                        "shortfall_points": round(100.0 * (e_t - e_run), 2),
                        "per_layer_effective": [round(v, 4) for v in e_l]})
        log(f"depth-ordered calibration, target e={e_t}: runtime effective {e_run:.4f} "
            f"({100.0 * (e_t - e_run):+.2f} points short)")
    return {"method": f"histogram, at most {ms_h} samples, {nb_h} bins, depth order on a chain of "
                      f"the {n_layers} layers (h_(l+1) = h_l + y_l, x_(l+1) = bf16(RMSNorm(h_(l+1)))), "
                      f"{n_cal} calibration tokens, {n_tok} held-out tokens",
            "alpha": round(alpha, 4), "targets": targets, "seconds": round(time.perf_counter() - t_cal0, 2)}


def proxy16_section(rot, taus, t_proj, alpha, t_stage1_int4, args):
    """The pages' precision ablation swaps the INT4 proxy for a 16-bit one at
    the same budget.  Here the 16-bit proxy is each rotated layer's own bf16
    W_up / W_gate (built on the GPU from the packed transposed weights): its
    Stage 1 over every input gives alpha_16, the allocator turns the same
    effective-sparsity targets at s1 = 0.7 into s2 (or reports them out of
    reach), and the reachable points and the headline configuration are
    timed."""
    import torch
    from free_ffn_activation_amd import prox
    d, f, n_layers = rot.d, rot.f, rot.n_layers
    K = max(1, args.steps)
    cfg = rot.cfg
    for L in rot.layers:
        L.add_proxy16()
        wt = L.w_upgate_t.view(f, 2, d)
        prox.prox_pack_proxy16(wt[:, 0, :].t().contiguous(), wt[:, 1, :].t().contiguous(), L)
    torch.cuda.synchronize()
    layers16 = [L.with_proxy_kind(prox.PROX_PROXY_W16) for L in rot.layers]
    o = Outs(d, f)

    def s1_16(tx_of):
        def fn(s):
            l, t = rot.at(s)
            prox.prox_ffn_decode_stages(layers16[l], rot.xs[l][t], tx_of(l), taus[l][1], o.y, o.mi, o.mc, o.ic, o.ws,
                                        prox.PROX_STAGE_PROXY)
        return fn

    spr = rot.steps_per_round
    t16_all = time_graph(s1_16(lambda l: 0.0), spr, K, "16-bit proxy: Stage 1 over every input", graph=not args.no_graph)
    alpha16 = t16_all / t_proj
    taus16 = rot.calibrate(cfg.keep_x, args.sparsity, layers16)
    t16_s1 = time_graph(s1_16(lambda l: taus16[l][0]), spr, K, "16-bit proxy: Stage 1 alone (keep_x 0.5)",
                        graph=not args.no_graph)

    def dec16(tl):
        def fn(s):
            l, t = rot.at(s)
            prox.prox_ffn_decode(layers16[l], rot.xs[l][t], tl[l][0], tl[l][1], o.y, o.mi, o.mc, o.ic, o.ws)
        return fn

    us16 = time_graph(dec16(taus16), spr, K, "16-bit proxy decode (keep_x 0.5, s2 0.7)", graph=not args.no_graph)
    kx16, ks16 = decode_counts(rot, taus16, layers16, o)
    mb16 = rot.tmean(4 * kx16 * f + 3 * ks16 * d * 2 + d * 2 + 4 * d + 4 * ks16, K)
    pts16 = []
    for e_t in (0.4, 0.5, 0.6, 0.7):
        try:
            s2p = prox.prox_budget_s2(e_t, 0.7, alpha16)
        except prox.ProxError as exc:
            if exc.status != prox.PROX_ERR_UNSUPPORTED:
                raise
            pts16.append({"e_target": e_t, "s1": 0.7, "reachable": False, "reason": str(exc)})
            continue
        tl = rot.calibrate(0.3, s2p, layers16)
        us_p = time_graph(dec16(tl), spr, K, f"16-bit proxy decode at e={e_t} s1=0.7 s2={s2p:.4f}",
                          graph=not args.no_graph)
        _kx_p, ks_p = decode_counts(rot, tl, layers16, o)
        pts16.append({"e_target": e_t, "s1": 0.7, "s2": round(s2p, 4), "reachable": True,
                      "us_per_layer": round(us_p, 3), "runtime_keep_s": round(rot.tmean(ks_p, K) / f, 4)})
    res = {"proxy": "the layer's own bf16 W_up / W_gate, row-major", "alpha": round(alpha16, 4),
           "alpha_int4": round(alpha, 4), "t_stage1_all_inputs_us": round(t16_all, 3),
           "t_stage1_us": round(t16_s1, 3), "t_stage1_int4_us": round(t_stage1_int4, 3),
           "us_per_layer": round(us16, 3), "required_MB": round(mb16 / 1e6, 3),
           "mean_k_x": round(rot.tmean(kx16, K), 1), "mean_k_s": round(rot.tmean(ks16, K), 1),
           "same_budget_s1_0.7": pts16, "proxy_bytes_per_layer": int(rot.layers[0].proxy_w16.numel())}
    log(f"16-bit proxy: alpha {alpha16:.3f} (INT4 {alpha:.3f}); Stage 1 {t16_s1:.2f} us (INT4 {t_stage1_int4:.2f}); "
        f"decode {us16:.2f} us at keep_x 0.5 / s2 0.7")
    for L in rot.layers:
        L.proxy_w16 = None
        L.desc = L._make_desc()
    del layers16
    torch.cuda.empty_cache()
    return res


def geglu_section(rot, args):
    """The same packed layers read as GeGLU (GELU-tanh gate), recalibrated at
    the headline keep / sparsity, timed over the same rotation."""
    from free_ffn_activation_amd import prox
    d, f = rot.d, rot.f
    K = max(1, args.steps)
    layers_g = [L.with_activation(prox.PROX_ACT_GELU_TANH) for L in rot.layers]
    taus_g = rot.calibrate(rot.cfg.keep_x, args.sparsity, layers_g)
    o = Outs(d, f)
    kx_g, ks_g = decode_counts(rot, taus_g, layers_g, o)

    def step_g(s):
        l, t = rot.at(s)
        prox.prox_ffn_decode(layers_g[l], rot.xs[l][t], taus_g[l][0], taus_g[l][1], o.y, o.mi, o.mc, o.ic, o.ws)

    us_g = time_graph(step_g, rot.steps_per_round, K, "GeGLU decode", graph=not args.no_graph)
    mb_g = rot.tmean(byte_model(kx_g, ks_g, d, f, 2)["step"], K)
    return {"activation": "gelu_tanh", "us_per_layer": round(us_g, 3), "required_MB": round(mb_g / 1e6, 3),
            "GBps": round(mb_g / (us_g * 1e-6) / 1e9, 1),
            "pct_hbm_roofline": round(100.0 * mb_g / (us_g * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
            "mean_k_x": round(rot.tmean(kx_g, K), 1), "mean_k_s": round(rot.tmean(ks_g, K), 1)}


def batch_union_counts(rot, taus, B, o):
    """Per (layer, group of B tokens): union of kept rows, union of kept
    channels, sum of k_s, mean k_x (the grouped path's algorithmic bytes)."""
    import torch
    from free_ffn_activation_amd import prox
    np = rot.np
    d, f, n_layers = rot.d, rot.f, rot.n_layers
    nb = rot.n_tok // B
    kxu = np.zeros((n_layers, nb), np.int64)
    ksu = np.zeros((n_layers, nb), np.int64)
    ks_sum = np.zeros((n_layers, nb), np.int64)
    kx_tok = np.zeros((n_layers, nb), np.float64)
    for l in range(n_layers):
        tx, ts = taus[l]
        for h in range(nb):
            xg = rot.x_all[l, B * h:B * h + B]
            prox.prox_ffn_decode(rot.layers[l], xg, tx, ts, o.y, o.mi, o.mc, o.ic, o.ws)
            torch.cuda.synchronize()
            xv = xg.view(torch.bfloat16).float().abs()
            kxu[l, h] = int((xv >= tx).any(dim=0).sum().item())
            cnt = o.mc.cpu().numpy()
            um = torch.zeros(f, dtype=torch.bool, device="cuda")
            for k in range(B):
                um[o.mi[k, :int(cnt[k])].long()] = True
            ksu[l, h] = int(um.sum().item())
            ks_sum[l, h] = int(cnt.sum())
            kx_tok[l, h] = float(o.ic.float().mean().item())
    by = {"step": kxu * f + 8 * kxu + 3 * ksu * d * 2 + B * (2 * d + 4 * d) + 4 * ks_sum,
          "stage1_proxy": kxu * f + 8 * kxu + B * 2 * d + B * f // 8,
          "stage2_upgate": 2 * ksu * d * 2 + B * 2 * d + 8 * ksu,
          "stage2_down": ksu * d * 2 + 8 * ksu + B * 4 * d}
    return kxu, ksu, ks_sum, kx_tok, by


def batch8_section(rot, taus, args):
    """Eight independent tokens per step through one layer (each token its
    own masks): the rotation's layers with their 16 tokens taken 8 at a time.
    Timed three ways on the same schedule: the grouped kernels (Stage 1 from
    the layers' channel-major proxy copies, every proxy row read once;
    Stage 2 reads the union of the tokens' channels once), the per-token
    kernels (PROX_STAGE_PER_TOKEN: each token reads its own rows and
    channels), torch's dense bf16 FFN at M = 8.  Required bytes use the union
    counts: K_x^U * d_ff + 8 K_x^U + 3 K_s^U * d * 2 + 8 (2d + 4d) +
    4 sum(k_s) (eight tokens that each keep half of the rows leave K_x^U
    within 1% of d)."""
    import numpy as np
    import torch
    from free_ffn_activation_amd import prox
    B = 8
    d, f, n_layers = rot.d, rot.f, rot.n_layers
    for L in rot.layers:
        L.add_proxy_qt()
    torch.cuda.synchronize()
    K = max(1, args.steps)
    nb = rot.n_tok // B
    sched_b = [(s % n_layers, (s // n_layers) % nb) for s in range(n_layers * nb)]
    nsb = len(sched_b)
    o = Outs(d, f, B)
    kxu, ksu, ks_sum, kx_tok, by = batch_union_counts(rot, taus, B, o)

    def bmean(a):
        return float(np.mean([a[sched_b[s % nsb]] for s in range(K)]))

    def b_step(stages):
        def fn(s):
            l, h = sched_b[s % nsb]
            tx, ts = taus[l]
            prox.prox_ffn_decode_stages(rot.layers[l], rot.x_all[l, B * h:B * h + B], tx, ts, o.y, o.mi, o.mc, o.ic,
                                        o.ws, stages)
        return fn

    us_grp = time_graph(b_step(7), nsb, K, "batch 8, grouped kernels", graph=not args.no_graph)
    us_pt = time_graph(b_step(7 | prox.PROX_STAGE_PER_TOKEN), nsb, K, "batch 8, per-token kernels",
                       graph=not args.no_graph)
    iso8 = [Outs(d, f, B) for _ in range(nsb)]

    def b_iso(stages):
        def fn(s):
            l, h = sched_b[s % nsb]
            tx, ts = taus[l]
            b = iso8[s % nsb]
            prox.prox_ffn_decode_stages(rot.layers[l], rot.x_all[l, B * h:B * h + B], tx, ts, b.y, b.mi, b.mc, b.ic,
                                        b.ws, stages)
        return fn

    for s in range(nsb):
        b_iso(7)(s)
    torch.cuda.synchronize()
    bits = [prox.PROX_STAGE_PROXY, prox.PROX_STAGE_UPGATE, prox.PROX_STAGE_DOWN]
    k8 = [time_graph(b_iso(bit), nsb, K, f"batch 8, {nm} alone", graph=not args.no_graph)
          for nm, bit in zip(STAGE_NAMES, bits)]
    del iso8
    dense8 = None
    if not args.no_dense:
        wug8 = [L.w_upgate_t.view(torch.bfloat16).view(2 * f, d) for L in rot.layers]
        wdn8 = [L.w_down.view(torch.bfloat16).view(f, d) for L in rot.layers]
        yb8 = torch.empty(B, d, dtype=torch.bfloat16, device="cuda")

        def dense8_fn(s):
            l, h = sched_b[s % nsb]
            xx = rot.x_all[l, B * h:B * h + B].view(torch.bfloat16)
            ug = torch.nn.functional.linear(xx, wug8[l])
            sv = ug[:, 0::2] * torch.nn.functional.silu(ug[:, 1::2])
            torch.matmul(sv, wdn8[l], out=yb8)

        for s in range(4):
            dense8_fn(s)
        torch.cuda.synchronize()
        dense8 = round(time_graph(dense8_fn, nsb, K, "batch 8, dense torch bf16", graph=not args.no_graph), 3)
    mb8 = bmean(by["step"])
    bk8 = [bmean(by[nm]) for nm in STAGE_NAMES]
    names8 = [nm + "_batch" for nm in STAGE_NAMES]
    dom8 = int(np.argmax(k8))
    ach8 = bk8[dom8] / (k8[dom8] * 1e-6) / 1e9
    key = traffic_key("qwen3_8b", d, f, rot.cfg.keep_x, args.sparsity, B)
    traffic8 = measured_traffic(names8[dom8], key, bk8[dom8])
    log(f"batch 8: grouped {us_grp:.2f} us/step ({mb8 / 1e6:.1f} MB union), per-token kernels {us_pt:.2f}, "
        f"dense torch {dense8}; kernels " + ", ".join(f"{STAGE_NAMES[i]} {k8[i]:.2f}" for i in range(3)))
    return {"batch": B, "us_per_step": round(us_grp, 3), "tokens_per_s": round(B / (us_grp * 1e-6), 1),
            "us_per_token": round(us_grp / B, 3), "timed_steps": K,
            "required_MB_union": round(mb8 / 1e6, 3), "GBps": round(mb8 / (us_grp * 1e-6) / 1e9, 1),
            "pct_hbm_roofline": round(100.0 * mb8 / (us_grp * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
            "mean_K_x_union": round(bmean(kxu), 1), "mean_K_s_union": round(bmean(ksu), 1),
            "mean_k_x_token": round(bmean(kx_tok), 1), "mean_k_s_token": round(bmean(ks_sum) / B, 1),
            "per_token_kernels_us_per_step": round(us_pt, 3), "dense_torch_bf16_us_per_step": dense8,
            "kernels": {names8[i]: {"us": round(k8[i], 3), "algorithmic_MB": round(bk8[i] / 1e6, 3),
                                    "GBps": round(bk8[i] / (k8[i] * 1e-6) / 1e9, 1)} for i in range(3)},
            "roofline": {"bound": "hbm", "kernel": names8[dom8], "achieved": round(ach8, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach8 / HBM_PEAK_GBPS, 4),
                         "traffic": traffic8["bytes_per_launch"] if traffic8 else None,
                         "traffic_detail": traffic8, "traffic_key": key},
            "schedule": f"{n_layers} layers x {nb} groups of 8 of their {rot.n_tok} tokens"}


def cpu_baseline(rot, taus, args):
    """The oracle as it stands (NumPy fp64, untuned) on the host cores: the
    headline layer's tokens in turn for about --cpu-seconds with every BLAS
    thread (median per decode), single-thread runs of a few of its tokens and
    of the tiny fp32 layer; and the agreement of the GPU's masks and y with
    the oracle's on the tokens decoded (in-band mask disagreements, y errors
    against the oracle's Stage 2 on the GPU's channel list)."""
    import numpy as np
    import threadpoolctl
    import torch

    import oracle
    import synth
    from free_ffn_activation_amd import prox
    tdir = os.path.join(ROOT, "tests")
    if tdir not in sys.path:
        sys.path.insert(0, tdir)
    from prox_gpu_util import band_compare, oracle_view, y_errors

    n_tok = rot.n_tok
    # the GPU's outputs for layer 0's tokens
    o = Outs(rot.d, rot.f)
    gpu = []
    for t in range(n_tok):
        prox.prox_ffn_decode(rot.layers[0], rot.xs[0][t], taus[0][0], taus[0][1], o.y, o.mi, o.mc, o.ic, o.ws)
        torch.cuda.synchronize()
        gpu.append((o.y.cpu().numpy()[0].astype(np.float64), o.mi.cpu().numpy()[0], int(o.mc.item()),
                    int(o.ic.item())))
    log("CPU oracle baseline: preparing layer 0 in fp64")
    ov = oracle_view(rot.host0)
    tx, ts = taus[0]

    def dec(x):
        return oracle.decode(x, ov["Wu"], ov["Wg"], ov["Wd"], ov["qu"], ov["su"], ov["qg"], ov["sg"], tx, ts)

    times, refs = [], {}
    t_start = time.perf_counter()
    tok = 0
    while time.perf_counter() - t_start < args.cpu_seconds or tok < n_tok:
        t1 = time.perf_counter()
        r = dec(ov["x_dec"][tok % n_tok])
        times.append(time.perf_counter() - t1)
        if tok < n_tok:
            refs[tok] = r
        tok += 1
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    with threadpoolctl.threadpool_limits(1):
        t1_times = []
        for t in range(3):
            t1 = time.perf_counter()
            dec(ov["x_dec"][t])
            t1_times.append(time.perf_counter() - t1)
    # agreement of the GPU's outputs with the oracle on layer 0's tokens
    in_band = out_band = 0
    kx_eq = True
    y_ma = y_rl = 0.0
    for t, ref in refs.items():
        yg, mig, mcg, icg = gpu[t]
        kx_eq = kx_eq and icg == ref["k_x"]
        oob, inb, _asc = band_compare(mig, mcg, ref["s_tilde"], ts)
        in_band += inb
        out_band += oob
        if mcg == ref["k_s"] and np.array_equal(mig[:mcg], ref["J"]):
            y_ref = ref["y"]
        else:  # the oracle's Stage 2 on the GPU's own channel list
            m = np.zeros(rot.f, bool)
            m[mig[:mcg]] = True
            y_ref = oracle.stage2(ov["x_dec"][t], ov["Wu"], ov["Wg"], ov["Wd"], m)["y"]
        ma, rl = y_errors(yg, y_ref)
        y_ma, y_rl = max(y_ma, ma), max(y_rl, rl)
    # the tiny fp32 layer, every thread and one thread
    tiny = synth.make_layer(synth.CONFIGS["tiny"], n_dec=1)
    tv = oracle_view(tiny)
    ttx, tts = oracle.calibrate(tv["x_cal"], tv["qu"], tv["su"], tv["qg"], tv["sg"], 0.5, 0.7)

    def tiny_runs(n):
        v = []
        for _ in range(n):
            t1 = time.perf_counter()
            oracle.decode(tv["x_dec"][0], tv["Wu"], tv["Wg"], tv["Wd"], tv["qu"], tv["su"], tv["qg"], tv["sg"], ttx,
                          tts)
            v.append(time.perf_counter() - t1)
        return v

    tiny_all = tiny_runs(101)
    with threadpoolctl.threadpool_limits(1):
        tiny_1 = tiny_runs(101)
    cfg = rot.cfg
    med = statistics.median(times) * 1e6
    res = {"value": round(med, 1), "unit": "us/layer", "cores": int(threads), "kind": "oracle",
           "sample": f"{len(times)} decode steps over the {n_tok} tokens of layer 0 ({cfg.name}, d={rot.d}, "
                     f"f={rot.f}), NumPy fp64 oracle, {sum(times):.1f} s of CPU work; median",
           "mean_us": round(statistics.mean(times) * 1e6, 1),
           "single_thread": {"qwen3_8b_layer_us_median": round(statistics.median(t1_times) * 1e6, 1),
                             "qwen3_8b_layer_runs": len(t1_times),
                             "tiny_layer_us_median": round(statistics.median(tiny_1) * 1e6, 1), "tiny_runs": 101},
           "tiny_layer_us_median": round(statistics.median(tiny_all) * 1e6, 1), "tiny_runs": 101,
           "gpu_vs_oracle": {"tokens": len(refs), "k_x_equal": bool(kx_eq), "mask_in_band": int(in_band),
                             "mask_out_of_band": int(out_band), "y_max_abs": float(f"{y_ma:.3e}"),
                             "y_rel_l2": float(f"{y_rl:.3e}"),
                             "band": "1e-3 relative of tau_s", "y_tolerance": "max-abs 2e-2, rel-L2 1e-2"}}
    log(f"CPU oracle: median {med:.0f} us/layer on {threads} threads ({len(times)} tokens); 1 thread "
        f"{res['single_thread']['qwen3_8b_layer_us_median']:.0f} us; tiny {res['tiny_layer_us_median']:.0f} us; "
        f"GPU vs oracle: in-band {in_band}, out-of-band {out_band}, y max-abs {y_ma:.2e} rel-L2 {y_rl:.2e}")
    return res


# ============================================================================ counter runs
GATHER_TABLE_ROWS = 1 << 21  # 128-byte rows of the gather cross-check table (256 MiB)


def gather_reference_rows() -> int:
    """Rows the gather cross-check selects: every other row on average."""
    return GATHER_TABLE_ROWS // 2


def pmc_copy(n_bytes: int, reps: int) -> None:
    """Device-to-device copies of a known size, the scale reference for the
    FETCH_SIZE / WRITE_SIZE counters; then, as a check that the scale holds
    for 128-byte gathers like the decode kernels' reads, a torch index_select
    of a random ascending half of the 128-byte rows of a 256 MiB table."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    g = torch.Generator().manual_seed(5)
    idx = torch.randperm(GATHER_TABLE_ROWS, generator=g)[:gather_reference_rows()].sort().values.to("cuda")
    table = torch.ones(GATHER_TABLE_ROWS, 64, dtype=torch.bfloat16, device="cuda")
    for _ in range(reps):
        out = torch.index_select(table, 0, idx)
    torch.cuda.synchronize()
    log(f"copied {n_bytes} bytes {reps} times; gathered {out.shape[0]} rows of 128 bytes {reps} times")


def pmc_run(args) -> None:
    """One eager decode pass over every (layer, token) of a workload's
    rotation (batch 1) or every (layer, group of 8 tokens) (batch 8), and the
    mean algorithmic bytes per launch of each decode kernel over exactly those
    launches (the counter runs average over the same launches)."""
    import numpy as np
    import synth
    cfg = synth.CONFIGS[args.pmc_run]
    n_layers = args.layers or {"qwen3_8b": 8, "qwen3_32b": 4}[args.pmc_run]
    rot = Rotation(cfg, n_layers, 16)
    taus = rot.calibrate(cfg.keep_x, args.sparsity)
    B = args.pmc_batch
    if B == 1:
        kx, ks = decode_counts(rot, taus)
        by = byte_model(kx, ks, rot.d, rot.f, 2)
        kernels = {nm: float(np.mean(by[nm])) for nm in STAGE_NAMES}
        launches = int(kx.size)
    else:
        for L in rot.layers:
            L.add_proxy_qt()
        _kxu, _ksu, _ks_sum, _kx_tok, by = batch_union_counts(rot, taus, B, Outs(rot.d, rot.f, B))
        kernels = {nm + "_batch": float(np.mean(by[nm])) for nm in STAGE_NAMES}
        launches = int(by["step"].size)
    meta = {"key": traffic_key(args.pmc_run, rot.d, rot.f, cfg.keep_x, args.sparsity, B),
            "launches": launches, "algorithmic_bytes_per_launch": kernels,
            "source_sha256": {k: kernel_source_hash(k) for k in kernels}}
    if args.pmc_meta:
        os.makedirs(os.path.dirname(os.path.abspath(args.pmc_meta)), exist_ok=True)
        with open(args.pmc_meta, "w") as fh:
            json.dump(meta, fh, indent=1)
    log(f"pmc run {args.pmc_run} batch {B}: {launches} decode calls; " +
        ", ".join(f"{k} {v / 1e6:.2f} MB" for k, v in kernels.items()))


def _counter_means(run_dir: str, counter: str) -> dict:
    """Mean counter value per dispatch of each kernel name in the rocprofv3
    counter_collection CSVs under run_dir (rows of one dispatch are added)."""
    per = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                k = (row["Kernel_Name"], row.get("Dispatch_Id") or row.get("Correlation_Id"))
                per[k] = per.get(k, 0.0) + float(row["Counter_Value"])
    by_name = {}
    for (name, _disp), v in per.items():
        by_name.setdefault(name, []).append(v)
    return {name: (sum(v) / len(v), len(v)) for name, v in by_name.items()}


def summarize_pmc(root: str) -> None:
    """Turns rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs into traffic records.

    Layout under root: copy_fetch/, copy_write/ (the --pmc-copy-mib 1024 runs)
    and for each tag: <tag>_fetch/, <tag>_write/ (the --pmc-run runs) and
    <tag>_meta.json (written by those runs).  Each counter is scaled by what
    it reads for the 1 GiB copy (bytes read resp. written); records merge into
    profiles/traffic.json by (kernel, workload, shape, keep fractions, batch),
    and a markdown table goes to stdout."""
    copy_bytes = 1 << 30
    cf = _counter_means(os.path.join(root, "copy_fetch"), "FETCH_SIZE")
    cw = _counter_means(os.path.join(root, "copy_write"), "WRITE_SIZE")
    cname = [n for n in cf if "copyBuffer" in n]
    wname = [n for n in cw if "copyBuffer" in n]
    if not cname or not wname:
        sys.exit("no copy-kernel counters found under " + root)
    fetch_kib_copy = max(cf[n][0] for n in cname)
    write_kib_copy = max(cw[n][0] for n in wname)
    fetch_factor = copy_bytes / (fetch_kib_copy * 1024.0)
    write_factor = copy_bytes / (write_kib_copy * 1024.0)
    # cross-check of the scale on a 128-byte-row gather of known size
    gname_f = [n for n in cf if "gather" in n.lower() or "indexselect" in n.lower().replace("_", "")]
    gname_w = [n for n in cw if "gather" in n.lower() or "indexselect" in n.lower().replace("_", "")]
    gather_check = None
    if gname_f and gname_w:
        n_rows = gather_reference_rows()
        g_read = n_rows * (128 + 8)   # the rows and their int64 indexes
        g_write = n_rows * 128
        gf = max(cf[n][0] for n in gname_f) * 1024.0 * fetch_factor
        gw = max(cw[n][0] for n in gname_w) * 1024.0 * write_factor
        gather_check = {"rows": n_rows, "row_bytes": 128, "algorithmic_read": g_read, "algorithmic_write": g_write,
                        "scaled_fetch": round(gf), "scaled_write": round(gw),
                        "fetch_ratio": round(gf / g_read, 4), "write_ratio": round(gw / g_write, 4)}
    try:
        with open(TRAFFIC_FILE) as fh:
            store = json.load(fh)
    except (OSError, ValueError):
        store = {}
    recs = store.get("records", [])
    lines = [f"Scale: a 1 GiB device copy reads FETCH_SIZE {fetch_kib_copy:.1f} KiB (factor x{fetch_factor:.4f}) "
             f"and WRITE_SIZE {write_kib_copy:.1f} KiB (factor x{write_factor:.4f}).", ""]
    lines += ["Check of the FETCH_SIZE scale on this library's own loads: every algorithmic byte a kernel does "
              "not write must be fetched at least once, so (algorithmic - written) / raw FETCH bytes is the "
              "smallest factor consistent with each launch (last column below).  A lower bound near the copy's "
              "factor (the contiguous 16 KB up/gate runs) pins the factor for these loads; a bound above it "
              "would expose an undercount.", ""]
    if gather_check:
        lines += [f"The scale depends on the request type: torch's index_select of {gather_check['rows']} rows of "
                  f"128 bytes (ascending random half of a 256 MiB table) reads raw FETCH_SIZE "
                  f"{gather_check['scaled_fetch'] / fetch_factor / 1e6:.2f} MB for {gather_check['algorithmic_read'] / 1e6:.2f} MB "
                  f"of rows and indexes, x{gather_check['fetch_ratio']:.3f} after the copy's factor (either that kernel "
                  f"fetches twice its bytes or its requests count at full size); its writes scale to "
                  f"x{gather_check['write_ratio']:.3f}.", ""]
    for meta_path in sorted(glob.glob(os.path.join(root, "*_meta.json"))):
        tag = os.path.basename(meta_path)[:-len("_meta.json")]
        with open(meta_path) as fh:
            meta = json.load(fh)
        fm = _counter_means(os.path.join(root, tag + "_fetch"), "FETCH_SIZE")
        wm = _counter_means(os.path.join(root, tag + "_write"), "WRITE_SIZE")
        key = meta["key"]
        lines += [f"### {tag}: {key}", "",
                  "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | algorithmic bytes | ratio "
                  "| FETCH factor lower bound |",
                  "|---|---|---|---|---|---|---|---|"]
        for kernel, alg in meta["algorithmic_bytes_per_launch"].items():
            pats = KERNELS[kernel][1]
            f_kib = sum(v[0] for n, v in fm.items() if any(p in n for p in pats))
            w_kib = sum(v[0] for n, v in wm.items() if any(p in n for p in pats))
            n_disp = min([v[1] for n, v in fm.items() if any(p in n for p in pats)] or [0])
            if n_disp == 0:
                continue
            fb = f_kib * 1024.0 * fetch_factor
            wb = w_kib * 1024.0 * write_factor
            # every algorithmic byte that is not written must be fetched at least once:
            # the smallest FETCH_SIZE factor consistent with this launch's raw count
            f_lb = (alg - wb) / (f_kib * 1024.0) if f_kib > 0 else None
            rec = {"kernel": kernel, **key, "source_sha256": meta["source_sha256"][kernel],
                   "dispatches": n_disp, "fetch_kib_raw": round(f_kib, 1), "write_kib_raw": round(w_kib, 1),
                   "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                   "hbm_bytes_per_launch": round(fb + wb), "algorithmic_bytes_per_launch": round(alg),
                   "ratio_to_algorithmic": round((fb + wb) / alg, 3),
                   "fetch_factor_lower_bound": None if f_lb is None else round(f_lb, 4)}
            recs = [r for r in recs if not (r.get("kernel") == kernel and all(r.get(k) == v for k, v in key.items()))]
            recs.append(rec)
            lines.append(f"| {kernel} | {n_disp} | {f_kib:.1f} | {w_kib:.1f} | {(fb + wb) / 1e6:.2f} MB | "
                         f"{alg / 1e6:.2f} MB | {(fb + wb) / alg:.3f} | "
                         f"{'-' if f_lb is None else f'{f_lb:.3f}'} |")
        lines.append("")
    store = {"_about": "HBM bytes per launch of the decode kernels from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE "
                       "runs (KiB per dispatch, mean over the dispatches of one pass over a workload's rotation), "
                       "scaled by the same counters on a 1 GiB device-to-device copy.  Keyed by kernel, workload, "
                       "shape, keep fractions and batch; source_sha256 covers the kernel's sources, prox_device.h and "
                       "prox_internal.h, and bench.py reports a record only while it matches.",
             "scale": {"copy_bytes": copy_bytes, "fetch_kib_read": round(fetch_kib_copy, 1),
                       "write_kib_read": round(write_kib_copy, 1), "fetch_factor": fetch_factor,
                       "write_factor": write_factor, "gather128_check": gather_check},
             "records": recs}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(store, fh, indent=1)
    print("\n".join(lines))


# ============================================================================ main
def main() -> int:
    args = parse()
    if args.gpus != 1:
        sys.exit(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
                 "(the decode path runs on a single GPU)")
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.pmc_copy_mib:
        pmc_copy(args.pmc_copy_mib << 20, 4)
        return 0
    if args.pmc_run:
        pmc_run(args)
        return 0

    import synth
    cfg = synth.CONFIGS[args.workload]
    n_layers = args.layers or {"qwen3_8b": 8, "qwen3_32b": 4}[args.workload]
    K = max(1, args.steps)
    records = [] if args.records else None

    rot = Rotation(cfg, n_layers, 16)
    taus = rot.calibrate(cfg.keep_x, args.sparsity)
    head, _kx, _ks = measure_decode(rot, taus, K, args.workload, cfg.keep_x, args.sparsity, args, records=records)
    log(f"headline: {head['us_per_layer']:.2f} us/layer, {head['required_MB_per_layer']:.2f} MB required, "
        f"{head['achieved_GBps']:.0f} GB/s ({head['pct_hbm_roofline']:.1f}% of 8 TB/s)")

    # streaming-copy context on this GPU
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2.0 * nbytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    budget = calibration = proxy16 = geglu = batch8 = None
    if not args.no_budget and cfg.dtype == "bf16":
        ap = {}
        budget = budget_section(rot, taus, ap, args)
        calibration = calibration_section(rot, ap["alpha"])
        proxy16 = proxy16_section(rot, taus, ap["t_proj"], ap["alpha"], head["kernels"]["stage1_proxy"]["us"], args)
        geglu = geglu_section(rot, args)
    if not args.no_batch and rot.n_tok % 8 == 0 and cfg.dtype == "bf16":
        batch8 = batch8_section(rot, taus, args)
    cpu = None if args.no_cpu_baseline else cpu_baseline(rot, taus, args)
    rot.free()

    configs = None
    if not args.no_configs and args.workload == "qwen3_8b":
        configs = {"stack36_sparsity_sweep": stack_sweep(args, records)}
        c32 = synth.CONFIGS["qwen3_32b"]
        rot32 = Rotation(c32, 4, 16)
        taus32 = rot32.calibrate(c32.keep_x, 0.7)
        r32, _, _ = measure_decode(rot32, taus32, args.config_steps, "qwen3_32b", c32.keep_x, 0.7, args,
                                   records=records)
        r32.update({"workload": "qwen3_32b", "d_model": c32.d_model, "d_ff": c32.d_ff, "layers_rotated": 4,
                    "keep_x": c32.keep_x, "sparsity_s": 0.7})
        configs["qwen3_32b"] = r32
        rot32.free()

    if records is not None:
        with open(args.records, "w") as fh:
            for r in records:
                fh.write(json.dumps(r) + "\n")
        log(f"wrote {len(records)} per-call records to {args.records}")

    out = {
        "metric": METRIC,
        "value": head["us_per_layer"],
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_layer"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}_ffn_layer_decode", "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "batch": 1, "keep_x": cfg.keep_x, "sparsity_s": args.sparsity,
                   "layers_rotated": n_layers, "tokens_per_layer": 16,
                   "timing": "eager" if args.no_graph else "hip_graph_replay"},
        "achieved_GBps": head["achieved_GBps"],
        "pct_hbm_roofline": head["pct_hbm_roofline"],
        "required_MB_per_layer": head["required_MB_per_layer"],
        "mean_k_x": head["mean_k_x"],
        "mean_k_s": head["mean_k_s"],
        "eager_us_per_layer": head["eager_us_per_layer"],
        "step_us": head["step_us"],
        "device_copy_GBps_read_plus_write": round(copy_gbps, 1),
        "kernels": head.get("kernels"),
        "dense_us_per_layer": head.get("dense_us_per_layer"),
        "roofline": head.get("roofline"),
        "cpu_baseline": cpu,
        "configs": configs,
        "budget": budget,
        "geglu": geglu,
        "calibration": calibration,
        "batch8": batch8,
        "proxy16": proxy16,
        "records_file": args.records,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
