"""Parity helpers: run the GPU pipeline through the C ABI and compare each
stage with the CPU oracle.

Comparison rule (values): |gpu - ref| <= tol * max(|ref|, |tau|), where tau is
that query's oracle h-th (for E) or k-th (for scores) value; the floor avoids
meaningless relative error on near-zero values that can never be selected.

When a query's list (its prefix, its MISA-dagger candidates or its MISA x
HISA candidates) holds no more than k entries, all are returned and no k-th
value separates them; likewise when the k-th value is a ReLU zero, every
positive value is returned.  tau is then the largest of them instead.

Comparison rule (selections): let band = {i : |ref_i - tau| <= tol*|tau|}.

Rounding allowance: where q_j . k cancels to near zero (or signed weights
cancel across heads), no accumulation order holds a relative bound; each
entry's bound and band are then at least EPS * M with M = sum_j |w_j|
(|q_j| . |k|), the size of the products the score adds up, and EPS = 2^-16
(fp32 accumulation of 128 products stays within about 2^-17 M).  M exceeds
the plain bound only for such cancelling entries, and is computed just for
the entries the plain rule rejects.
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
            k=None, kprime=None, m=None, device="cuda:0"):
    """Run the requested stages through the C ABI; returns numpy outputs.

    "step" (decode problems with bf16/fp8 inputs only) runs misa_decode_step
    on a copy of the pooled cache whose last block was overwritten, so the
    step must rebuild it; its outputs carry the prefix "s_".  "hisa" runs
    misa_hisa_score_topk with m blocks on the routed heads; its outputs carry
    the prefix "h"."""
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
    if "route" in stages or "score" in stages or "dagger" in stages or "hisa" in stages:
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
    if "hisa" in stages:
        hws = torch.empty(max(1, misa.misa_hisa_workspace_bytes(shp, h, m, k)), dtype=torch.uint8,
                          device=dev)
        hb = torch.empty((p.batch, p.T, m), dtype=torch.int32, device=dev)
        hbs = torch.empty((p.batch, p.T, m), dtype=torch.float32, device=dev)
        idx = torch.empty((p.batch, p.T, k), dtype=torch.int32, device=dev)
        sc = torch.empty((p.batch, p.T, k), dtype=torch.float32, device=dev)
        misa.misa_hisa_score_topk(shp, h, m, k, q, qs, w, pooled, kk, ks, out["heads"], hb, hbs,
                                  idx, sc, hws)
        out["hb"], out["hbs"], out["h_idx"], out["h_scores"] = hb, hbs, idx, sc
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
    """The k-th largest value (the last one when fewer than k): the centre of
    the selection tie band."""
    k = min(k, len(vals))
    return float(np.partition(vals, len(vals) - k)[len(vals) - k])


def value_tau(vals: np.ndarray, k: int) -> float:
    """tau of the value comparison: the k-th largest value.  A list of at most
    k values is selected whole, and when the k-th value is a ReLU zero every
    positive value is selected: either way no value separates selected from
    rejected entries, and tau is then the largest magnitude (the scale of
    the list)."""
    v = kth_value(vals, k)
    return float(np.max(np.abs(vals))) if len(vals) <= k or v == 0.0 else v


EPS = 2.0 ** -16


def gross(seq, q, w, heads):
    """keys -> M = sum over the (valid) heads of |w_j| (|q_j| . |k|): the size
    of the products a score adds up (the rounding allowance's scale)."""
    hs = np.asarray([j for j in np.asarray(heads).tolist() if 0 <= j < len(w)], dtype=np.int64)
    qa = np.abs(np.asarray(q)[hs]) * np.abs(np.asarray(w)[hs])[:, None]  # [h, d]
    qsum = qa.sum(axis=0)  # sum_j |w_j| |q_j|  (d,)
    K = seq.K

    def m(keys):
        keys = np.asarray(keys, dtype=np.int64)
        return np.abs(K[keys]) @ qsum
    return m


def gross_E(seq, q, w, pos: int, B: int):
    """Per head j, M of E_j (Eq. 7): |w_j| / M_t times the sum over the
    complete blocks of |q_j| . |p_b| plus, for a partial last block, the mean
    over its keys of |q_j| . |k_s| (the size of the products E adds up)."""
    n = pos + 1
    full, Mt = n // B, (n + B - 1) // B
    qa = np.abs(np.asarray(q))  # [H, d]
    acc = qa @ np.abs(np.asarray(seq.pooled)[:full]).sum(axis=0) if full else np.zeros(qa.shape[0])
    if n % B:
        acc = acc + qa @ np.abs(seq.K[full * B:n]).mean(axis=0)
    return np.abs(np.asarray(w)) * acc / Mt


def gross_G(seq, q, w, pos: int, B: int):
    """Per block b, M of the block score G_b: sum_j |w_j| |q_j| . |p_b|, the
    partial last block taking the mean over its keys of the same with |k_s|."""
    n = pos + 1
    full = n // B
    qa = (np.abs(np.asarray(q)) * np.abs(np.asarray(w))[:, None]).sum(axis=0)  # (d,)
    out = np.abs(np.asarray(seq.pooled)[:full]) @ qa
    if n % B:
        out = np.append(out, np.abs(seq.K[full * B:n]).mean(axis=0) @ qa)
    return out


def check_values(gpu, ref, tol, tau, what="", mag=None):
    """mag: callable (positions in these arrays) -> M of those entries (the
    rounding allowance EPS * M), or None."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lim = tol * np.maximum(np.abs(ref), abs(tau))
    over = np.abs(gpu - ref) > lim
    if mag is not None and over.any():
        pos = np.nonzero(over)[0]
        lim = lim.copy()
        lim[pos] = np.maximum(lim[pos], EPS * mag(pos))
    bad = np.abs(gpu - ref) > lim
    assert not bad.any(), (
        f"{what}: {bad.sum()} values out of tolerance; first at {np.argmax(bad)}: "
        f"gpu={gpu[bad][0]!r} ref={ref[bad][0]!r} tau={tau!r}")


def check_selection(gpu_sel, ref_sel, ref_score_of, tau, tol, what="", mag_of=None):
    """gpu_sel/ref_sel: 1-D index arrays (-1 = padding); ref_score_of: callable
    index -> oracle score (double); mag_of: callable index -> M of that index
    (the rounding allowance), or None."""
    g = [int(i) for i in gpu_sel if i >= 0]
    r = [int(i) for i in ref_sel if i >= 0]
    assert len(g) == len(set(g)), f"{what}: duplicate indices in the GPU selection"
    G, R = set(g), set(r)
    assert len(G) == len(R), f"{what}: |gpu| = {len(G)} != |ref| = {len(R)}"
    for i in G ^ R:
        s = ref_score_of(i)
        band = tol * abs(tau)
        if abs(s - tau) > band and mag_of is not None:
            band = max(band, EPS * float(mag_of(i)))
        assert abs(s - tau) <= band, (
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
        ME = gross_E(seq, q, w, pos, p.B)
        check_values(gpu["E"][b, t], E_ref, tol, value_tau(E_ref, h), f"E[{b},{t}]", lambda ps: ME[ps])
        gh = gpu["heads"][b, t]
        assert np.all(np.diff(gh) > 0), f"heads[{b},{t}] not ascending: {gh}"
        out["head_swaps"] = check_selection(gh, heads_ref, lambda j: E_ref[j], tau, tol,
                                            f"heads[{b},{t}]", lambda j: ME[j])
    if "idx" in gpu:
        heads = gpu["heads"][b, t]
        I = seq.scores(pos, q, w, heads)
        M = gross(seq, q, w, heads)
        k = gpu["idx"].shape[2]
        ref = oracle.topk(I, k)
        tau = kth_value(I, k)
        out["tok_swaps"] = check_selection(gpu["idx"][b, t], ref, lambda s: I[s], tau, tol,
                                           f"idx[{b},{t}]", M)
        sel = gpu["idx"][b, t]
        valid = sel >= 0
        check_values(gpu["scores"][b, t][valid], I[sel[valid]], tol, value_tau(I, k), f"scores[{b},{t}]",
                     lambda ps: M(sel[valid][ps]))
    return out


def check_query_dense(op: OracleProblem, gpu: dict, b: int, t: int, tol: float):
    seq = op.seq(b)
    pos = op.pos(t)
    k = gpu["d_idx"].shape[2]
    r = seq.dense(pos, op.q[b, t], op.w[b, t], k)
    I = r["scores"]
    M = gross(seq, op.q[b, t], op.w[b, t], np.arange(op.p.H))
    tau = kth_value(I, k)
    sw = check_selection(gpu["d_idx"][b, t], r["idx"], lambda s: I[s], tau, tol, f"dense[{b},{t}]", M)
    sel = gpu["d_idx"][b, t]
    valid = sel >= 0
    check_values(gpu["d_scores"][b, t][valid], I[sel[valid]], tol, value_tau(I, k),
                 f"dense scores[{b},{t}]", lambda ps: M(sel[valid][ps]))
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
    M = gross(seq, q, w, heads)
    tau = kth_value(I, kp)
    sw1 = check_selection(gpu["cand"][b, t], oracle.topk(I, kp), lambda s: I[s], tau, tol,
                          f"cand[{b},{t}]", M)
    sw2 = check_rerank(op, gpu["cand"][b, t], gpu["r_idx"][b, t], gpu["r_scores"][b, t], b, t, tol)
    return {"cand_swaps": sw1, "rerank_swaps": sw2}


def check_rerank(op: OracleProblem, cand, r_idx, r_scores, b: int, t: int, tol: float):
    """Eq. (12) for query (b, t) given its candidate list (entries < 0 are
    padding): the selection within the tie band and the returned scores."""
    seq = op.seq(b)
    q, w = op.q[b, t], op.w[b, t]
    kp = len(cand)
    k = len(r_idx)
    valid_c = cand[cand >= 0]
    if len(valid_c) == 0:
        assert np.all(r_idx == -1) and np.all(r_scores == -np.inf), f"rerank[{b},{t}]: no candidate"
        return 0
    idx_ref, sc_ref = oracle.rerank(seq.K, q, w, cand, k)
    # Eq. (1) score of every candidate, from the oracle (rerank keeping all).
    all_idx, all_sc = oracle.rerank(seq.K, q, w, cand, kp)
    dense_of = {int(i): float(v) for i, v in zip(all_idx, all_sc) if i >= 0}
    Mall = gross(seq, q, w, np.arange(op.p.H))
    sel = r_idx
    assert all(int(s) in dense_of for s in sel if s >= 0), f"rerank[{b},{t}]: index not a candidate"
    tau2 = float(sc_ref[min(k, len(valid_c)) - 1])
    tau2_v = value_tau(np.asarray([dense_of[int(i)] for i in valid_c if int(i) in dense_of]), k)
    sw2 = check_selection(sel, idx_ref, lambda s: dense_of[s], tau2, tol, f"rerank[{b},{t}]", Mall)
    v = sel >= 0
    check_values(r_scores[v], [dense_of[int(s)] for s in sel[v]], tol, tau2_v,
                 f"rerank scores[{b},{t}]", lambda ps: Mall(sel[v][ps]))
    assert np.all(r_scores[~v] == -np.inf), f"rerank[{b},{t}]: padding scores not -inf"
    return sw2


def check_query_hisa(op: OracleProblem, gpu: dict, b: int, t: int, tol: float):
    """MISA x HISA for query (b, t): the blocks against the oracle's block
    scores G (all heads), then the top-k given the GPU's heads and blocks.

    G sums w * ReLU over heads and may cancel when weights are negative, so
    its tolerance scale also takes the same sum with |w| (the size of the
    terms that were added)."""
    p = op.p
    seq = op.seq(b)
    pos = op.pos(t)
    q, w = op.q[b, t], op.w[b, t]
    m = gpu["hb"].shape[2]
    G = seq.block_scores(pos, q, w)
    Gabs = seq.block_scores(pos, q, np.abs(w))
    Mt = len(G)
    gb = gpu["hb"][b, t]
    nb = min(m, Mt)
    assert np.all(gb[nb:] == -1), f"hb[{b},{t}]: padding {gb[nb:]}"
    sel = gb[:nb]
    assert np.all(sel >= 0) and np.all(sel < Mt), f"hb[{b},{t}]: blocks out of range {sel}"
    assert np.all(np.diff(sel) > 0), f"hb[{b},{t}] not ascending: {sel}"
    tau = kth_value(G, m)
    scale = np.maximum(np.abs(G), np.abs(tau))
    scale = np.maximum(scale, Gabs)
    allow = np.maximum(tol * scale, EPS * gross_G(seq, q, w, pos, p.B))  # (rounding allowance)
    G_sel = set(int(i) for i in sel)
    ref_sel = set(int(i) for i in oracle.topk(G, m) if i >= 0)
    assert len(G_sel) == len(ref_sel), f"hb[{b},{t}]: {len(G_sel)} blocks, oracle {len(ref_sel)}"
    for j in G_sel ^ ref_sel:
        assert abs(G[j] - tau) <= allow[j], (
            f"hb[{b},{t}]: block {j} (G {G[j]!r}, |w| sum {Gabs[j]!r}) differs outside the tie "
            f"band around {tau!r}")
    hbs = gpu["hbs"][b, t][:nb].astype(np.float64)
    bad = np.abs(hbs - G[sel]) > allow[sel]
    assert not bad.any(), f"hbs[{b},{t}]: {bad.sum()} block scores out of tolerance"
    assert np.all(gpu["hbs"][b, t][nb:] == -np.inf)
    # Tokens: the oracle's Eq. (9) over the GPU's blocks with the GPU's heads.
    heads = gpu["heads"][b, t]
    I = seq.scores(pos, q, w, heads)
    M = gross(seq, q, w, heads)
    toks = np.concatenate([np.arange(j * p.B, min((j + 1) * p.B, pos + 1)) for j in sel])
    k = gpu["h_idx"].shape[2]
    cs = I[toks]
    ref = toks[oracle.topk(cs, k)[: min(k, len(toks))]]
    tau2 = kth_value(cs, k)
    # At most k candidates (every one is taken) or a ReLU-zero k-th value: no
    # selection boundary among the values, so their error scale is the size
    # of the query's scores (fp8 codes are accumulated in fp32 at their own
    # scale).
    tau_v = value_tau(cs, k)
    gi = gpu["h_idx"][b, t]
    tokset = set(int(s) for s in toks)
    assert all(int(s) in tokset for s in gi if s >= 0), f"h_idx[{b},{t}]: token outside the blocks"
    sw = check_selection(gi, ref, lambda s: I[s], tau2, tol, f"h_idx[{b},{t}]", M)
    v = gi >= 0
    check_values(gpu["h_scores"][b, t][v], I[gi[v]], tol, tau_v, f"h_scores[{b},{t}]",
                 lambda ps: M(gi[v][ps]))
    assert np.all(gi[~v] == -1) and np.all(gpu["h_scores"][b, t][~v] == -np.inf)
    return {"block_swaps": len(G_sel ^ ref_sel), "tok_swaps": sw}
