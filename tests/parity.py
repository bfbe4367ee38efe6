"""Parity helpers: run the GPU pipeline through the C ABI and compare each
stage with the CPU oracle.

Comparison rule (values): |gpu - ref| <= tol * max(|ref|, |tau|), where tau is
that query's oracle h-th (for E) or k-th (for scores) value; the floor avoids
meaningless relative error on near-zero values that can never be selected.

Comparison rule (selections): let band = {i : |ref_i - tau| <= tol*|tau|}.
The GPU set and the oracle set must have the same size, agree exactly outside
the band, and differ only inside it.  Later stages are compared with the
oracle fed the GPU's own (already checked) upstream output, so a legitimate
near-tie swap does not cascade.

Tolerances: 1e-3 relative for fp32/bf16 inputs (fp32 accumulation), 2e-2 for
fp8 inputs.
"""

from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import oracle
import synth

TOL = {synth.F32: 1e-3, synth.BF16: 1e-3, synth.FP8_E4M3: 2e-2}
ORACLE_DTYPE = {synth.F32: oracle.F32, synth.BF16: oracle.BF16, synth.FP8_E4M3: oracle.FP8_E4M3}
_POOL = concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 4))


def pmap(fn, items):
    """Run oracle calls over independent queries on a thread pool (ctypes
    releases the GIL, so the single-threaded oracle runs in parallel)."""
    return list(_POOL.map(fn, items))


# ------------------------------------------------------------------ oracle data


class OracleProblem:
    """Decoded inputs of one problem, per sequence, for the oracle."""

    def __init__(self, x: synth.Inputs):
        self.x = x
        self.p = x.problem
        self._seqs = {}
        dt = ORACLE_DTYPE[self.p.dtype]
        p = self.p
        qraw = x.raw_numpy("q").reshape(p.batch * p.T, p.H * p.d)
        qs = x.q_scale.numpy().reshape(-1) if p.dtype == synth.FP8_E4M3 else None
        self.q = oracle.decode(qraw, dt, qs).reshape(p.batch, p.T, p.H, p.d)
        self.w = x.w.double().numpy()

    def seq(self, b: int) -> oracle.Sequence:
        if b not in self._seqs:
            p = self.p
            dt = ORACLE_DTYPE[p.dtype]
            ks = self.x.k_scale[b].numpy() if p.dtype == synth.FP8_E4M3 else None
            K = oracle.decode(self.x.raw_numpy("k")[b], dt, ks)
            self._seqs[b] = oracle.Sequence(K, p.B)
        return self._seqs[b]

    def pos(self, t: int) -> int:
        return self.p.L - self.p.T + t


# ------------------------------------------------------------------ GPU run


def run_gpu(x: synth.Inputs, stages=("pool", "route", "score", "dense", "dagger", "step"), h=None,
            k=None, kprime=None, device="cuda:0"):
    """Run the requested stages through the C ABI; returns numpy outputs.

    "step" (decode problems with bf16/fp8 inputs only) runs misa_decode_step
    on a copy of the pooled cache whose last block was overwritten, so the
    step must rebuild it; its outputs carry the prefix "s_"."""
    import torch

    import long_context_pool_amd as misa

    p = x.problem
    h = h or p.h
    k = k or p.k
    kprime = kprime or p.kprime
    dev = torch.device(device)
    q, kk, w = x.q.to(dev), x.k.to(dev), x.w.to(dev)
    fp8 = p.dtype == synth.FP8_E4M3
    qs = x.q_scale.to(dev) if fp8 else None
    ks = x.k_scale.to(dev) if fp8 else None
    shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
    ws = torch.empty(max(1, misa.misa_workspace_bytes(shp, h, k, kprime or k)), dtype=torch.uint8,
                     device=dev)
    out = {}
    pooled = torch.empty((p.batch, p.M, p.d), dtype=torch.float32, device=dev)
    misa.misa_pool_keys(shp, kk, ks, pooled)
    out["pooled"] = pooled
    if "route" in stages or "score" in stages or "dagger" in stages:
        heads = torch.empty((p.batch, p.T, h), dtype=torch.int32, device=dev)
        E = torch.empty((p.batch, p.T, p.H), dtype=torch.float32, device=dev)
        misa.misa_route(shp, h, q, qs, w, pooled, kk, ks, heads, E, ws)
        out["heads"], out["E"] = heads, E
    if "score" in stages:
        idx = torch.empty((p.batch, p.T, k), dtype=torch.int32, device=dev)
        sc = torch.empty((p.batch, p.T, k), dtype=torch.float32, device=dev)
        misa.misa_score_topk(shp, h, k, q, qs, w, kk, ks, out["heads"], idx, sc, ws)
        out["idx"], out["scores"] = idx, sc
    if "dense" in stages:
        idx = torch.empty((p.batch, p.T, k), dtype=torch.int32, device=dev)
        sc = torch.empty((p.batch, p.T, k), dtype=torch.float32, device=dev)
        misa.dsa_index_dense(shp, k, q, qs, w, kk, ks, idx, sc, ws)
        out["d_idx"], out["d_scores"] = idx, sc
    if "dagger" in stages and kprime:
        cand = torch.empty((p.batch, p.T, kprime), dtype=torch.int32, device=dev)
        csc = torch.empty((p.batch, p.T, kprime), dtype=torch.float32, device=dev)
        misa.misa_score_topk(shp, h, kprime, q, qs, w, kk, ks, out["heads"], cand, csc, ws)
        idx = torch.empty((p.batch, p.T, k), dtype=torch.int32, device=dev)
        sc = torch.empty((p.batch, p.T, k), dtype=torch.float32, device=dev)
        misa.misa_rerank(shp, kprime, k, q, qs, w, kk, ks, cand, idx, sc, ws)
        out["cand"], out["cand_scores"], out["r_idx"], out["r_scores"] = cand, csc, idx, sc
    if "step" in stages and p.T == 1 and p.dtype != synth.F32:
        sp = pooled.clone()
        sp[:, p.M - 1].fill_(7.0)
        heads = torch.empty((p.batch, 1, h), dtype=torch.int32, device=dev)
        E = torch.empty((p.batch, 1, p.H), dtype=torch.float32, device=dev)
        idx = torch.empty((p.batch, 1, k), dtype=torch.int32, device=dev)
        sc = torch.empty((p.batch, 1, k), dtype=torch.float32, device=dev)
        misa.misa_decode_step(shp, h, k, q, qs, w, sp, kk, ks, heads, E, idx, sc, ws)
        out["s_pooled"], out["s_heads"], out["s_E"], out["s_idx"], out["s_scores"] = (
            sp, heads, E, idx, sc)
    torch.cuda.synchronize()
    return {name: v.cpu().numpy() for name, v in out.items()}


def step_view(gpu: dict) -> dict:
    """The misa_decode_step outputs under the names check_query_misa reads."""
    return {"E": gpu["s_E"], "heads": gpu["s_heads"], "idx": gpu["s_idx"],
            "scores": gpu["s_scores"]}


# ------------------------------------------------------------------ comparators


def kth_value(vals: np.ndarray, k: int) -> float:
    """The k-th largest value (the last one when fewer than k)."""
    k = min(k, len(vals))
    return float(np.partition(vals, len(vals) - k)[len(vals) - k])


def check_values(gpu, ref, tol, tau, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lim = tol * np.maximum(np.abs(ref), abs(tau))
    bad = np.abs(gpu - ref) > lim
    assert not bad.any(), (
        f"{what}: {bad.sum()} values out of tolerance; first at {np.argmax(bad)}: "
        f"gpu={gpu[bad][0]!r} ref={ref[bad][0]!r} tau={tau!r}")


def check_selection(gpu_sel, ref_sel, ref_score_of, tau, tol, what=""):
    """gpu_sel/ref_sel: 1-D index arrays (-1 = padding); ref_score_of: callable
    index -> oracle score (double)."""
    g = [int(i) for i in gpu_sel if i >= 0]
    r = [int(i) for i in ref_sel if i >= 0]
    assert len(g) == len(set(g)), f"{what}: duplicate indices in the GPU selection"
    G, R = set(g), set(r)
    assert len(G) == len(R), f"{what}: |gpu| = {len(G)} != |ref| = {len(R)}"
    for i in G ^ R:
        s = ref_score_of(i)
        assert abs(s - tau) <= tol * abs(tau), (
            f"{what}: index {i} (ref score {s!r}) differs outside the tie band around {tau!r}")
    return len(G ^ R)


def check_query_misa(op: OracleProblem, gpu: dict, b: int, t: int, tol: float):
    """Route, routed score + top-k for query (b, t), stage-conditional."""
    p = op.p
    seq = op.seq(b)
    pos = op.pos(t)
    q, w = op.q[b, t], op.w[b, t]
    out = {}
    if "E" in gpu:
        E_ref, heads_ref = seq.route(pos, q, w, gpu["heads"].shape[2])
        h = gpu["heads"].shape[2]
        tau = kth_value(E_ref, h)
        check_values(gpu["E"][b, t], E_ref, tol, tau, f"E[{b},{t}]")
        gh = gpu["heads"][b, t]
        assert np.all(np.diff(gh) > 0), f"heads[{b},{t}] not ascending: {gh}"
        out["head_swaps"] = check_selection(gh, heads_ref, lambda j: E_ref[j], tau, tol,
                                            f"heads[{b},{t}]")
    if "idx" in gpu:
        heads = gpu["heads"][b, t]
        I = seq.scores(pos, q, w, heads)
        k = gpu["idx"].shape[2]
        ref = oracle.topk(I, k)
        tau = kth_value(I, k)
        out["tok_swaps"] = check_selection(gpu["idx"][b, t], ref, lambda s: I[s], tau, tol,
                                           f"idx[{b},{t}]")
        sel = gpu["idx"][b, t]
        valid = sel >= 0
        check_values(gpu["scores"][b, t][valid], I[sel[valid]], tol, tau, f"scores[{b},{t}]")
    return out


def check_query_dense(op: OracleProblem, gpu: dict, b: int, t: int, tol: float):
    seq = op.seq(b)
    pos = op.pos(t)
    k = gpu["d_idx"].shape[2]
    r = seq.dense(pos, op.q[b, t], op.w[b, t], k)
    I = r["scores"]
    tau = kth_value(I, k)
    sw = check_selection(gpu["d_idx"][b, t], r["idx"], lambda s: I[s], tau, tol, f"dense[{b},{t}]")
    sel = gpu["d_idx"][b, t]
    valid = sel >= 0
    check_values(gpu["d_scores"][b, t][valid], I[sel[valid]], tol, tau, f"dense scores[{b},{t}]")
    return {"dense_swaps": sw, "dense_idx": r["idx"]}


def check_query_dagger(op: OracleProblem, gpu: dict, b: int, t: int, tol: float):
    """The candidate pass (Eq. 11) given the GPU heads, then the rerank
    (Eq. 12) given the GPU candidates."""
    seq = op.seq(b)
    pos = op.pos(t)
    q, w = op.q[b, t], op.w[b, t]
    heads = gpu["heads"][b, t]
    kp = gpu["cand"].shape[2]
    k = gpu["r_idx"].shape[2]
    I = seq.scores(pos, q, w, heads)
    tau = kth_value(I, kp)
    sw1 = check_selection(gpu["cand"][b, t], oracle.topk(I, kp), lambda s: I[s], tau, tol,
                          f"cand[{b},{t}]")
    cand = gpu["cand"][b, t]
    idx_ref, sc_ref = oracle.rerank(seq.K, q, w, cand, k)
    valid_c = cand[cand >= 0]
    # Eq. (1) score of every candidate, from the oracle (rerank keeping all).
    all_idx, all_sc = oracle.rerank(seq.K, q, w, cand, kp)
    dense_of = {int(i): float(v) for i, v in zip(all_idx, all_sc) if i >= 0}
    sel = gpu["r_idx"][b, t]
    assert all(int(s) in dense_of for s in sel if s >= 0), f"rerank[{b},{t}]: index not a candidate"
    tau2 = float(sc_ref[min(k, len(valid_c)) - 1])
    sw2 = check_selection(sel, idx_ref, lambda s: dense_of[s], tau2, tol, f"rerank[{b},{t}]")
    v = sel >= 0
    check_values(gpu["r_scores"][b, t][v], [dense_of[int(s)] for s in sel[v]], tol, tau2,
                 f"rerank scores[{b},{t}]")
    return {"cand_swaps": sw1, "rerank_swaps": sw2}
