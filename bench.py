"""Benchmark of the MISA indexer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

The default workload is the largest: a 128K-token prefill chunk in fp8 (T =
8192 queries ending an L = 131072 causal prefix, H = 64, h = 8, B = 128,
k = 2048) with MISA-dagger (k' = 8192 candidates re-ranked by all heads).

A step is one pass of the hot path over one batch of synthetic input:
  decode (T = 1): misa_decode_step -- refresh the pooled key of the block
                  holding the newest token (the pooled-key cache update),
                  route, routed score + top-k in two kernels
                  [-> rerank when the workload has k'];
  prefill:        pool all keys -> route -> routed score + top-k [-> rerank].
`value` is the whole step of the workload (MISA-dagger when it has k').  For
such workloads the one-stage MISA step (routed top-k straight to k, no
re-rank) is timed too, and for bf16/fp8 workloads the MISA x HISA step
(pool -> route -> the top m = 8192 / B blocks by the head-summed router
affinities -> routed top-k inside them).  The dense DSA indexer (all heads,
same library) is timed the same way for the MISA-vs-DSA speedups.  Inputs are resident in HBM
before timing starts; several input sets are rotated so that the decode
workloads stream their keys from HBM instead of the 256 MB last-level cache.

Prints one JSON line (metric/value = scored (query, token) pairs per second).
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scored (query,token) pairs/s + MISA-vs-dense-DSA speedup, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "long_context_pool_amd", "csrc")


def source_sha() -> str:
    """Hash of the kernel sources and of the build script (its flags shape
    the kernels too)."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    files.append(os.path.join(os.path.dirname(CSRC), "build.py"))
    for path in files:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5",
                    help="c1..c5 (default c5, the 128K fp8 prefill with MISA-dagger)")
    ap.add_argument("--L", type=int, default=0,
                    help="override the workload's context length (a sweep point, not a headline "
                         "configuration: the line's workload name then carries _L<L>)")
    ap.add_argument("--T", type=int, default=0,
                    help="override the workload's queries per sequence (likewise; _T<T>)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-1stage", action="store_true",
                    help="skip the one-stage MISA leg of workloads with k' (profiling the main call alone)")
    ap.add_argument("--hisa-m", type=int, default=-1,
                    help="blocks per query of the MISA x HISA leg (-1: 8192 / B, 4k candidates "
                         "at k = 2048; 0: skip the leg)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate wall time of the oracle baseline")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="after timing, copy BYTES device-to-device (profiler counter calibration)")
    return ap.parse_args()


class Runner:
    """Device buffers of several input sets and the per-step call sequence."""

    def __init__(self, x, n_sets, stream):
        import torch

        import long_context_pool_amd as misa
        import synth

        self.misa = misa
        self.p = p = x.problem
        self.stream = stream
        dev = torch.device("cuda:0")
        fp8 = p.dtype == synth.FP8_E4M3
        self.shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
        kp = p.kprime or p.k
        self.ws = torch.empty(misa.misa_workspace_bytes(self.shp, p.h, p.k, kp), dtype=torch.uint8,
                              device=dev)
        self.sets = []
        with torch.cuda.stream(stream):
            for i in range(n_sets):
                s = {
                    "q": x.q.to(dev), "k": x.k.to(dev), "w": x.w.to(dev),
                    "qs": x.q_scale.to(dev) if fp8 else None,
                    "ks": x.k_scale.to(dev) if fp8 else None,
                    "pooled": torch.empty((p.batch, p.M, p.d), dtype=torch.float32, device=dev),
                }
                misa.misa_pool_keys(self.shp, s["k"], s["ks"], s["pooled"], stream)
                self.sets.append(s)
            self.heads = torch.empty((p.batch, p.T, p.h), dtype=torch.int32, device=dev)
            self.cand = torch.empty((p.batch, p.T, kp), dtype=torch.int32, device=dev)
            self.idx = torch.empty((p.batch, p.T, p.k), dtype=torch.int32, device=dev)
            self.didx = torch.empty((p.batch, p.T, p.k), dtype=torch.int32, device=dev)
            self.idx1 = torch.empty((p.batch, p.T, p.k), dtype=torch.int32, device=dev)
            self.idxh = torch.empty((p.batch, p.T, p.k), dtype=torch.int32, device=dev)
        self.decode = p.T == 1
        self.hisa_m = 0
        self.hws = None

    def set_hisa(self, m):
        import torch

        self.hisa_m = m
        self.hws = torch.empty(self.misa.misa_hisa_workspace_bytes(self.shp, self.p.h, m, self.p.k),
                               dtype=torch.uint8, device="cuda:0")

    def _pool_route(self, s):
        """Pooling (Eq. (4)) and routing (Eq. (7)-(8)) of a prefill step."""
        m, p, st = self.misa, self.p, self.stream
        if p.T <= 8:
            # Multi-query decode: the pooled cache only changes in the
            # blocks holding the T newest keys.
            b0 = (p.L - p.T) // p.B
            m.misa_pool_keys_range(self.shp, b0, p.M - b0, s["k"], s["ks"], s["pooled"], st)
        else:
            m.misa_pool_keys(self.shp, s["k"], s["ks"], s["pooled"], st)
        m.misa_route(self.shp, p.h, s["q"], s["qs"], s["w"], s["pooled"], s["k"], s["ks"],
                     self.heads, None, self.ws, st)

    def misa_step(self, i, ev=None):
        """One MISA pass on input set i; ev = (before, after) events around the
        dominant call (decode: misa_decode_step; prefill: the routed score +
        top-k)."""
        m, p, s, st = self.misa, self.p, self.sets[i % len(self.sets)], self.stream
        out = self.cand if p.kprime else self.idx
        if self.decode:
            if ev:
                ev[0].record(st)
            m.misa_decode_step(self.shp, p.h, p.kprime or p.k, s["q"], s["qs"], s["w"], s["pooled"],
                               s["k"], s["ks"], self.heads, None, out, None, self.ws, st)
            if ev:
                ev[1].record(st)
        else:
            self._pool_route(s)
            if ev:
                ev[0].record(st)
            m.misa_score_topk(self.shp, p.h, p.kprime or p.k, s["q"], s["qs"], s["w"], s["k"],
                              s["ks"], self.heads, out, None, self.ws, st)
            if ev:
                ev[1].record(st)
        if p.kprime:
            m.misa_rerank(self.shp, p.kprime, p.k, s["q"], s["qs"], s["w"], s["k"], s["ks"],
                          self.cand, self.idx, None, self.ws, st)

    def misa_1stage_step(self, i, ev=None):
        """MISA without the re-rank (Eq. (7)-(10) with k), for workloads
        whose headline step is MISA-dagger; ev brackets misa_score_topk."""
        m, p, s, st = self.misa, self.p, self.sets[i % len(self.sets)], self.stream
        if self.decode:
            if ev:
                ev[0].record(st)
            m.misa_decode_step(self.shp, p.h, p.k, s["q"], s["qs"], s["w"], s["pooled"], s["k"],
                               s["ks"], self.heads, None, self.idx1, None, self.ws, st)
            if ev:
                ev[1].record(st)
            return
        self._pool_route(s)
        if ev:
            ev[0].record(st)
        m.misa_score_topk(self.shp, p.h, p.k, s["q"], s["qs"], s["w"], s["k"], s["ks"], self.heads,
                          self.idx1, None, self.ws, st)
        if ev:
            ev[1].record(st)

    def hisa_step(self, i, ev=None):
        """MISA x HISA: pooling and routing, then the top-m blocks by the
        head-summed affinities and the routed top-k inside them; ev brackets
        misa_hisa_score_topk."""
        m, p, s, st = self.misa, self.p, self.sets[i % len(self.sets)], self.stream
        self._pool_route(s)
        if ev:
            ev[0].record(st)
        m.misa_hisa_score_topk(self.shp, p.h, self.hisa_m, p.k, s["q"], s["qs"], s["w"],
                               s["pooled"], s["k"], s["ks"], self.heads, None, None, self.idxh,
                               None, self.hws, st)
        if ev:
            ev[1].record(st)

    def dense_step(self, i, ev=None):
        m, p, s, st = self.misa, self.p, self.sets[i % len(self.sets)], self.stream
        if ev:
            ev[0].record(st)
        m.dsa_index_dense(self.shp, p.k, s["q"], s["qs"], s["w"], s["k"], s["ks"], self.didx, None,
                          self.ws, st)
        if ev:
            ev[1].record(st)


def time_steps(fn, steps, warmup, stream):
    """Run warmup, then exactly `steps` timed steps with nothing else on the
    stream, then `steps` more with events around the dominant call.  Returns
    (ms per step of the timed run, mean ms of the bracketed call, host ms per
    step spent submitting the timed run, {10, 50, 90: percentile of the
    bracketed call's ms})."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    host_ms = (time.perf_counter() - t0) * 1e3 / steps  # submission only
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / steps
    # Per-call durations, in a second run: events recorded between calls
    # would add their own gaps to the timed run.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        fn(i, evs[i])
    torch.cuda.synchronize()
    calls = sorted(a.elapsed_time(b) for a, b in evs)
    call_ms = sum(calls) / steps
    pct = {q: calls[min(len(calls) - 1, int(q / 100 * len(calls)))] for q in (10, 50, 90)}
    return step_ms, call_ms, host_ms, pct


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload.

    The sample is every sequence of a decode batch, or 32 evenly spaced
    queries of a prefill.  Three legs, each in whole passes over (part of)
    the sample until its share of budget_s has gone:
      * the method of the workload (MISA: route + routed score + top-k,
        plus the re-rank for MISA-dagger) on a thread pool of host cores
        (ctypes releases the GIL; at most 16 threads) -- the reported value;
      * the same on one core, over the first 4 queries of the sample;
      * dense DSA (Eq. (1)-(2)) on the thread pool."""
    import concurrent.futures

    import numpy as np

    import oracle
    import synth

    p = x.problem
    odt = {synth.F32: oracle.F32, synth.BF16: oracle.BF16, synth.FP8_E4M3: oracle.FP8_E4M3}[p.dtype]
    cores = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count())
    if p.T == 1:
        sample = [(b, 0) for b in range(p.batch)]
    else:
        sample = [(0, int(t)) for t in np.linspace(0, p.T - 1, 32).round()]
    seqs = {}
    qraw = x.raw_numpy("q")
    for b in sorted({b for b, _ in sample}):
        ks = x.k_scale[b].numpy() if p.dtype == synth.FP8_E4M3 else None
        seqs[b] = oracle.Sequence(oracle.decode(x.raw_numpy("k")[b], odt, ks), p.B)

    def query_inputs(bt):
        b, t = bt
        qs = x.q_scale[b, t:t + 1].numpy() if p.dtype == synth.FP8_E4M3 else None
        q = oracle.decode(qraw[b, t].reshape(1, -1), odt, qs).reshape(p.H, p.d)
        return q, x.w[b, t].double().numpy()

    inputs = {bt: query_inputs(bt) for bt in sample}

    def misa_one(bt):
        b, t = bt
        q, w = inputs[bt]
        pos = p.L - p.T + t
        r = seqs[b].misa(pos, q, w, p.h, p.kprime or p.k)
        if p.kprime:
            oracle.rerank(seqs[b].K, q, w, r["idx"], p.k)
        return pos + 1

    def dense_one(bt):
        b, t = bt
        q, w = inputs[bt]
        pos = p.L - p.T + t
        seqs[b].dense(pos, q, w, p.k)
        return pos + 1

    def timed(fn, items, threads, budget):
        pairs, passes = 0, 0
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            t0 = time.perf_counter()
            while True:
                pairs += sum(ex.map(fn, items))
                passes += 1
                dt = time.perf_counter() - t0
                if dt >= budget:
                    return pairs / dt, passes, dt

    v_n, passes, dt = timed(misa_one, sample, cores, budget_s * 0.6)
    v_1, passes_1, _ = timed(misa_one, sample[:4], 1, budget_s * 0.2)
    v_d, passes_d, _ = timed(dense_one, sample, cores, budget_s * 0.2)
    what = "route + routed score + top-k" + (" + rerank" if p.kprime else "")
    desc = (f"{passes} pass(es) over {len(sample)} queries "
            f"({'every sequence' if p.T == 1 else 'evenly spaced'}) of the workload: {what}; "
            f"one core: {passes_1} pass(es) over the first 4; dense DSA: {passes_d} pass(es)")
    return {"value": v_n, "unit": "pairs/s", "cores": cores, "kind": "oracle", "sample": desc,
            "seconds": round(dt, 3), "one_core_value": v_1, "dense_value": v_d,
            "dense_one_core_estimate": v_d / cores, "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count()}


def traffic_from_profile(kernel, workload, sha):
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != sha:
        return None
    return d.get("bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the MISA indexer path is single-GPU "
              "(no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    p = synth.CONFIGS[args.workload]
    wl_name = args.workload
    if args.L or args.T:
        L, T = args.L or p.L, args.T or p.T
        if not 1 <= T <= L:
            print(f"--L {L} / --T {T}: need 1 <= T <= L", file=sys.stderr)
            sys.exit(2)
        tag = (f"_L{L}" if args.L else "") + (f"_T{T}" if args.T else "")
        p = dataclasses.replace(p, L=L, T=T, name=f"{p.name}{tag}")
        wl_name = f"{args.workload}{tag}"
    x = synth.generate(p)
    set_bytes = (x.q.numel() * x.q.element_size() + x.k.numel() * x.k.element_size() +
                 p.batch * p.M * p.d * 4)
    n_sets = max(2, min(16, math.ceil(768 * 2**20 / set_bytes)))
    stream = torch.cuda.Stream()  # default priority
    r = Runner(x, n_sets, stream)
    torch.cuda.synchronize()

    m_step, m_call, m_host, m_pct = time_steps(r.misa_step, args.steps, args.warmup, stream)
    pairs = p.pairs
    res_1stage = None
    if p.kprime and not args.no_1stage:
        s_step, s_call, _, _ = time_steps(r.misa_1stage_step, args.steps, args.warmup, stream)
        res_1stage = {"value": pairs / (s_step / 1e3), "ms_per_step": s_step,
                      "score_topk_call_ms": s_call, "k": p.k}
    res_hisa = None
    hisa_m = (8192 // p.B) if args.hisa_m < 0 else args.hisa_m
    if hisa_m > 0 and p.dtype != synth.F32:
        r.set_hisa(hisa_m)
        h_step, h_call, _, _ = time_steps(r.hisa_step, args.steps, args.warmup, stream)
        res_hisa = {"m": hisa_m, "value": pairs / (h_step / 1e3), "ms_per_step": h_step,
                    "hisa_call_ms": h_call, "k": p.k}
    res_dense = None
    if not args.no_dense:
        d_step, d_call, _, _ = time_steps(r.dense_step, args.steps, args.warmup, stream)
        res_dense = {"value": pairs / (d_step / 1e3), "ms_per_step": d_step}
    torch.cuda.synchronize()

    # Recall of the dense top-k (sets; last step's outputs, same input set).
    def recall_of(sel):
        a, b = sel.cpu().numpy(), r.didx.cpu().numpy()
        tot = 0
        for bi in range(p.batch):
            for t in range(p.T):
                tot += len(np.intersect1d(a[bi, t], b[bi, t]))
        return tot / (p.batch * p.T * p.k)

    import numpy as np

    recall = None
    if res_dense is not None:
        r.misa_step(0)
        r.dense_step(0)
        if res_1stage is not None:
            r.misa_1stage_step(0)
        if res_hisa is not None:
            r.hisa_step(0)
        torch.cuda.synchronize()
        recall = recall_of(r.idx)
        if res_1stage is not None:
            res_1stage["recall_vs_dense"] = recall_of(r.idx1)
            res_1stage["speedup_vs_dense"] = res_dense["ms_per_step"] / res_1stage["ms_per_step"]
        if res_hisa is not None:
            res_hisa["recall_vs_dense"] = recall_of(r.idxh)
            res_hisa["speedup_vs_dense"] = res_dense["ms_per_step"] / res_hisa["ms_per_step"]

    e = {synth.F32: 4, synth.BF16: 2, synth.FP8_E4M3: 1}[p.dtype]
    dtype = {synth.F32: "f32", synth.BF16: "bf16", synth.FP8_E4M3: "fp8"}[p.dtype]
    sha = source_sha()
    kp = p.kprime or p.k
    if p.T == 1:
        # Decode step: every key (and fp8 key scale), the pooled-key cache, the
        # query heads and w are read once; the k' (or k) indices are written.
        per_seq = (p.L * p.d * e + (p.L * 4 if e == 1 else 0) + p.M * p.d * 4 + p.H * p.d * e
                   + p.H * 4 + kp * 4)
        alg_bytes = p.batch * per_seq
        achieved = alg_bytes / (m_call * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "kernel": ("misa_decode_step call: decode_step_kernel + decode_select_kernel"
                           if p.batch >= 8 else
                           "misa_decode_step call: step_route_kernel + decode_score_kernel + "
                           "decode_select_kernel"),
                "algorithmic_bytes": alg_bytes,
                "traffic": traffic_from_profile("misa_decode_step", wl_name, sha)}
    else:
        flops = 2 * p.h * p.d * pairs
        achieved = flops / (m_call * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[dtype]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak,
                "kernel": "misa_score_topk call: prefill_clear_kernel + prefill_score_kernel + "
                          "prefill_select_kernel + prefill_repair_kernel",
                "algorithmic_flops": flops,
                "traffic": traffic_from_profile("misa_score_topk", wl_name, sha)}
    roof["call_ms"] = m_call
    roof["call_ms_p10_p50_p90"] = [m_pct[10], m_pct[50], m_pct[90]]

    if args.calibrate_copy:
        n = args.calibrate_copy // 16 * 16
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": pairs / (m_step / 1e3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": p.name, "batch": p.batch, "L": p.L, "T": p.T, "H": p.H, "h": p.h,
                   "d": p.d, "B": p.B, "k": p.k, "kprime": p.kprime, "pairs_per_step": pairs,
                   "input_sets": n_sets, "parallelism": "single-gpu"},
        "method": "MISA-dagger (k' candidates re-ranked)" if p.kprime else "MISA",
        "dense_dsa": res_dense,
        "speedup_vs_dense": (res_dense["ms_per_step"] / m_step) if res_dense else None,
        "recall_vs_dense": recall,
        "misa_1stage": res_1stage,
        "misa_x_hisa": res_hisa,
        "host_submit_ms_per_step": m_host,
        "source_sha": sha,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
