"""GPU parity: every stage of the HIP path against the CPU oracle, through the
C ABI, on seeded synthetic inputs.

Small problems (several tiles, ragged tails, partial router blocks) are
checked on every query.  The full-size workloads are checked on every
sequence (decode) or on one query of every 32-query workgroup tile (prefill:
128 and 256 queries) for the router, the routed top-k, the MISA-dagger
candidate pass and the re-rank; dense DSA (8x the oracle work) on every
sequence or on a fixed sample.  Every query of every workload is checked for
the properties that hold at any size, and the recall of the dense top-k is
asserted against a floor.  Exact-integer inputs force bit-identical scores
and heavy ties on every path (prefill, decode, decode step, multi-query).
Tolerances and the tie-band rule are in tests/parity.py.
"""

from __future__ import annotations

import dataclasses
import os
import sys

import numpy as np
import pytest
import torch

import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


SMALL = {
    "c1_tiny_fp32": synth.C1,
    "bf16_ragged": synth.small("bf16_ragged", batch=2, L=3000, T=70, H=64, h=8, B=64, k=300,
                               kprime=700, dtype=synth.BF16, needles=8, seed=21),
    "fp8_ragged": synth.small("fp8_ragged", batch=1, L=2500, T=50, H=64, h=8, B=128, k=256,
                              kprime=600, dtype=synth.FP8_E4M3, needles=8, seed=22),
    "h32_decode": synth.small("h32_decode", batch=4, L=5000, T=1, H=32, h=8, B=128, k=512,
                              kprime=1024, dtype=synth.BF16, needles=16, seed=23),
    "fp8_decode": synth.small("fp8_decode", batch=3, L=4100, T=1, H=64, h=8, B=64, k=400,
                              kprime=900, dtype=synth.FP8_E4M3, needles=12, seed=26),
    # Decode batches of 8 and more take the single-kernel step (one
    # workgroup per 256/batch of the chip per sequence); batch 12 leaves
    # some waves with no keys.
    "bf16_decode_b8": synth.small("bf16_decode_b8", batch=8, L=3000, T=1, H=64, h=8, B=64, k=300,
                                  kprime=700, dtype=synth.BF16, needles=8, seed=27),
    "fp8_decode_b12": synth.small("fp8_decode_b12", batch=12, L=2100, T=1, H=32, h=8, B=128, k=200,
                                  kprime=500, dtype=synth.FP8_E4M3, needles=6, seed=28),
    # Long rows at batch 8: each select workgroup covers 4608 keys (two
    # 4096-score chunks), and the last workgroup of a row has none.
    "bf16_decode_b8_long": synth.small("bf16_decode_b8_long", batch=8, L=140000, T=1, H=16, h=4, B=128,
                                       k=256, kprime=512, dtype=synth.BF16, needles=8, seed=29),
    # Decode edge shapes: a context shorter than k (every key, -1 padding) in
    # one partial block, and a two-block context with the newest block partial.
    "decode_lt_k": synth.small("decode_lt_k", batch=3, L=50, T=1, H=64, h=8, B=64, k=64, kprime=96,
                               dtype=synth.BF16, needles=2, seed=30),
    "decode_two_blocks": synth.small("decode_two_blocks", batch=9, L=100, T=1, H=64, h=8, B=64, k=32,
                                     kprime=48, dtype=synth.FP8_E4M3, needles=2, seed=31),
    # Multi-query decode (2 <= T <= 8 queries at the end of each sequence):
    # head bands of 8, 8, 4 and 16 rows; 1, 4, 1 and 3 row tiles.
    "mq_bf16_t2": synth.small("mq_bf16_t2", batch=3, L=3000, T=2, H=64, h=8, B=64, k=300, kprime=700,
                              dtype=synth.BF16, needles=6, seed=32),
    "mq_fp8_t8": synth.small("mq_fp8_t8", batch=2, L=2500, T=8, H=32, h=8, B=128, k=256, kprime=512,
                             dtype=synth.FP8_E4M3, needles=6, seed=33),
    "mq_h4_t4": synth.small("mq_h4_t4", batch=2, L=1500, T=4, H=64, h=4, B=64, k=100, kprime=200,
                            dtype=synth.BF16, needles=4, seed=34),
    "mq_h16_t3": synth.small("mq_h16_t3", batch=2, L=2000, T=3, H=64, h=16, B=64, k=128, kprime=256,
                             dtype=synth.FP8_E4M3, needles=4, seed=35),
    # Small k against L: the prefill threshold is sampled in several chunks
    # (the kept top sample values carried between them).
    "sample_chunks_bf16": synth.small("sample_chunks_bf16", batch=1, L=16384, T=100, H=64, h=8, B=64,
                                      k=64, kprime=160, dtype=synth.BF16, needles=8, seed=38),
    "sample_chunks_fp8": synth.small("sample_chunks_fp8", batch=2, L=12000, T=40, H=64, h=8, B=128,
                                     k=48, kprime=96, dtype=synth.FP8_E4M3, needles=8, seed=39),
    # k = 64 of a 64K prefix in eight splits: four sample chunks, and no plan
    # meets the repair bound, so some queries also go to the repair path.
    "sample_chunks4_fp8": synth.small("sample_chunks4_fp8", batch=1, L=65536, T=64, H=64, h=8, B=128,
                                      k=64, kprime=128, dtype=synth.FP8_E4M3, needles=8, seed=40),
    # 2048 queries: the re-rank gives each query one workgroup and takes its
    # top-k in the same workgroup (64 or 32 heads, fp8 or bf16).
    "fused_rerank_fp8": synth.small("fused_rerank_fp8", batch=1, L=4096, T=2048, H=64, h=8, B=128,
                                    k=128, kprime=512, dtype=synth.FP8_E4M3, needles=16, seed=36),
    "fused_rerank_bf16_h32": synth.small("fused_rerank_bf16_h32", batch=2, L=3000, T=1024, H=32, h=8,
                                         B=64, k=100, kprime=300, dtype=synth.BF16, needles=8, seed=37),
    "t_eq_l": synth.small("t_eq_l", batch=1, L=200, T=200, H=64, h=8, B=64, k=64, kprime=96,
                          dtype=synth.BF16, needles=0, seed=24),
    # The pages' own block size, B = 1024: five blocks, the last partial
    # (router partial blocks larger than the staged rows), prefill and a
    # batch-8 fp8 decode step (newest-block mean over up to 1024 keys).
    "b1024_prefill": synth.small("b1024_prefill", batch=1, L=4500, T=40, H=64, h=8, B=1024, k=256,
                                 kprime=600, dtype=synth.BF16, needles=6, seed=46),
    "b1024_decode_fp8": synth.small("b1024_decode_fp8", batch=8, L=3900, T=1, H=32, h=8, B=1024, k=200,
                                    kprime=400, dtype=synth.FP8_E4M3, needles=4, seed=47),
    "b1_h16": synth.small("b1_h16", batch=1, L=700, T=9, H=64, h=16, B=1, k=100, kprime=200,
                          dtype=synth.F32, needles=4, seed=25),
}
SMALL["c1_tiny_fp32"] = synth.small("c1", kprime=512)  # C1 plus a MISA-dagger stage


@pytest.fixture(scope="module", params=list(SMALL))
def small_case(request):
    p = SMALL[request.param]
    _log(f"[gpu] small case {request.param}: {p}")
    x = synth.generate(p)
    gpu = parity.run_gpu(x)
    return request.param, x, gpu, parity.OracleProblem(x)


def _all_queries(p):
    return [(b, t) for b in range(p.batch) for t in range(p.T)]


def test_small_pool(small_case):
    name, x, gpu, op = small_case
    p = x.problem
    for b in range(p.batch):
        ref = op.seq(b).pooled
        scale = np.abs(op.seq(b).K).max()
        np.testing.assert_allclose(gpu["pooled"][b], ref, rtol=1e-5, atol=1e-6 * scale)


def test_small_route_and_score(small_case):
    name, x, gpu, op = small_case
    p = x.problem
    tol = parity.TOL[p.dtype]
    res = parity.pmap(lambda bt: parity.check_query_misa(op, gpu, *bt, tol), _all_queries(p))
    hs = sum(r["head_swaps"] for r in res)
    ts = sum(r["tok_swaps"] for r in res)
    _log(f"[gpu] {name}: {len(res)} queries, head swaps in band {hs}, token swaps in band {ts}")


def _check_step(op, gpu, qs, tol, name):
    """misa_decode_step against the oracle: the rebuilt last pooled block,
    then route and routed top-k of each query in qs."""
    p = op.p
    for b in {b for b, _ in qs}:
        ref = op.seq(b).pooled
        got = gpu["s_pooled"][b]
        np.testing.assert_allclose(got[p.M - 1], ref[p.M - 1], rtol=1e-5, atol=1e-6 * np.abs(ref).max(),
                                   err_msg=f"{name}: decode step pooled block {p.M - 1} of seq {b}")
        np.testing.assert_array_equal(got[: p.M - 1], gpu["pooled"][b, : p.M - 1])
    view = parity.step_view(gpu)
    res = parity.pmap(lambda bt: parity.check_query_misa(op, view, *bt, tol), qs)
    _log(f"[gpu] {name}: decode step ok on {len(qs)} queries; head swaps "
         f"{sum(r['head_swaps'] for r in res)}, token swaps {sum(r['tok_swaps'] for r in res)}")


def test_small_decode_step(small_case):
    name, x, gpu, op = small_case
    p = x.problem
    if "s_idx" not in gpu:
        pytest.skip("misa_decode_step covers decode (T = 1) with bf16/fp8 inputs")
    _check_step(op, gpu, _all_queries(p), parity.TOL[p.dtype], name)


def test_small_dense(small_case):
    name, x, gpu, op = small_case
    p = x.problem
    tol = parity.TOL[p.dtype]
    res = parity.pmap(lambda bt: parity.check_query_dense(op, gpu, *bt, tol), _all_queries(p))
    # Recall of the dense top-k by MISA (GPU sets).
    rec = []
    for (b, t), r in zip(_all_queries(p), res):
        d = set(int(i) for i in gpu["d_idx"][b, t] if i >= 0)
        m = set(int(i) for i in gpu["idx"][b, t] if i >= 0)
        rec.append(len(d & m) / max(1, len(d)))
    _log(f"[gpu] {name}: MISA recall of dense top-k = {np.mean(rec):.4f}")


def test_small_dagger(small_case):
    name, x, gpu, op = small_case
    p = x.problem
    tol = parity.TOL[p.dtype]
    res = parity.pmap(lambda bt: parity.check_query_dagger(op, gpu, *bt, tol), _all_queries(p))
    rec = []
    for b, t in _all_queries(p):
        d = set(int(i) for i in gpu["d_idx"][b, t] if i >= 0)
        m = set(int(i) for i in gpu["r_idx"][b, t] if i >= 0)
        rec.append(len(d & m) / max(1, len(d)))
    _log(f"[gpu] {name}: MISA-dagger recall of dense top-k = {np.mean(rec):.4f}; "
         f"cand swaps {sum(r['cand_swaps'] for r in res)}, rerank swaps {sum(r['rerank_swaps'] for r in res)}")


# MISA x HISA: (case, m).  m B below k (the list padded up to k), every
# block of the early queries (M_t <= m), the fused re-rank select (2048
# queries), 32 heads, a context shorter than one block.
HISA = {
    "bf16_ragged": 8, "fp8_ragged": 4, "h32_decode": 8, "t_eq_l": 2, "mq_fp8_t8": 4,
    "fused_rerank_fp8": 4, "decode_lt_k": 1, "sample_chunks4_fp8": 2, "fp8_decode_b12": 3,
}
HISA_PAD = {"bf16_ragged": 4, "fp8_decode_b12": 1}  # m B = 256 < k = 300; 128 < 200 (decode)
# Many blocks per query: the top-m search over G held in registers (up to
# 64 per lane: 2048 < M_t <= 4096) and re-read from memory (M_t > 4096); and
# every key equal (all block scores tie: the search has no differing bit).
HISA_EXTRA = {
    "hisa_b2_mid": (synth.small("hisa_b2_mid", batch=1, L=6000, T=5, H=64, h=8, B=2, k=100,
                                kprime=None, dtype=synth.BF16, needles=4, seed=42), 256),
    "hisa_b1_long": (synth.small("hisa_b1_long", batch=1, L=5000, T=3, H=32, h=4, B=1, k=64,
                                 kprime=None, dtype=synth.FP8_E4M3, needles=4, seed=43), 512),
    "hisa_equal_keys": (synth.small("hisa_equal_keys", batch=2, L=1000, T=6, H=64, h=8, B=64, k=50,
                                    kprime=None, dtype=synth.BF16, needles=0, seed=44), 3),
    # 2048 queries (the re-rank takes each query's top-k in its own
    # workgroup) with m B = 128 < k = 200: the list is padded up to k.
    "hisa_fused_pad": (synth.small("hisa_fused_pad", batch=1, L=3000, T=2048, H=32, h=8, B=64, k=200,
                                   kprime=None, dtype=synth.FP8_E4M3, needles=4, seed=45), 2),
}


@pytest.mark.parametrize("name,m", list(HISA.items()) + [(n + "/pad", m) for n, m in HISA_PAD.items()]
                         + [(n, m) for n, (_, m) in HISA_EXTRA.items()])
def test_small_hisa(name, m):
    p = HISA_EXTRA[name][0] if name in HISA_EXTRA else SMALL[name.split("/")[0]]
    _log(f"[gpu] hisa {name} m={m}: {p}")
    x = synth.generate(p)
    if name == "hisa_equal_keys":
        x.k[:] = x.k[:, :1].clone()
    gpu = parity.run_gpu(x, stages=("pool", "route", "hisa"), m=m)
    op = parity.OracleProblem(x)
    res = parity.pmap(lambda bt: parity.check_query_hisa(op, gpu, *bt, parity.TOL[p.dtype]),
                      _all_queries(p))
    _log(f"[gpu] hisa {name}: {len(res)} queries; block swaps in band "
         f"{sum(r['block_swaps'] for r in res)}, token swaps {sum(r['tok_swaps'] for r in res)}")


def test_hisa_with_every_block_is_the_routed_top_k():
    """m >= M: the block stage keeps every block, so the selection is the
    routed top-k of misa_score_topk (both exact on integer inputs)."""
    p = synth.small("hisa_all", batch=2, L=1000, T=20, H=64, h=8, B=64, k=100, kprime=None,
                    dtype=synth.BF16, needles=0, seed=41)
    x = synth.generate(p, exact_ints=True)
    gpu = parity.run_gpu(x, stages=("pool", "route", "score", "hisa"), m=p.M)
    for name, idx, sc in (("h", gpu["h_idx"], gpu["h_scores"]), ("misa", gpu["idx"], gpu["scores"])):
        o = np.argsort(idx, axis=-1, kind="stable")
        gpu[name + "_sorted"] = (np.take_along_axis(idx, o, -1), np.take_along_axis(sc, o, -1))
    np.testing.assert_array_equal(gpu["h_sorted"][0], gpu["misa_sorted"][0])
    np.testing.assert_array_equal(gpu["h_sorted"][1], gpu["misa_sorted"][1])
    for t in range(p.T):
        Mt = (p.L - p.T + t + p.B) // p.B
        assert np.all(gpu["hb"][:, t, :Mt] == np.arange(Mt)) and np.all(gpu["hb"][:, t, Mt:] == -1)


# ---------------------------------------------------------------- random shapes
#
# Seeded random problems over the shape space the entry points accept:
# decode and prefill, bf16 / fp8 (fp32 now and then), 16-64 heads and 1-16
# routed, block sizes that are and are not powers of two (1 to 256), lists
# shorter than k, k' above k, and MISA x HISA with m B up to the limit.
# Every stage of every query is checked against the oracle.


def _random_problem(seed: int):
    rng = np.random.default_rng(9000 + seed)
    dtype = (synth.F32 if seed % 7 == 6 else (synth.BF16, synth.FP8_E4M3)[seed % 2])
    H = int(rng.choice([16, 32, 64]))
    h = int(rng.integers(1, min(H, 16) + 1))
    u = rng.random()
    T = 1 if u < 0.4 else (int(rng.integers(2, 9)) if u < 0.6 else int(rng.integers(9, 301)))
    batch = int(rng.integers(1, 9)) if T <= 8 else int(rng.integers(1, 3))
    B = int(rng.choice([1, 2, 7, 16, 64, 100, 128, 256, 1024]))
    u = rng.random()
    if seed >= 300 and T <= 4 and u < 0.3:
        L = int(rng.integers(40000, 120001))  # (long sweeps only) long decode rows
    elif u < 0.15 and T <= 16:
        L = int(rng.integers(6000, 40001))  # several key splits, long decode rows
    elif u < 0.3:
        L = int(rng.integers(T, T + 200))  # context about as long as the query chunk
    else:
        L = int(rng.integers(max(T, 2), 6001))
    kmax = 8192 if seed >= 300 else 1024
    k = int(rng.integers(1, min(L, kmax) + 1)) if rng.random() < 0.8 else int(rng.integers(L, L + 300))
    k = max(1, min(k, 8192))
    kprime = int(rng.integers(k + 1, min(4 * k, 8192) + 2)) if rng.random() < 0.7 and k < 8192 else None
    needles = int(rng.integers(0, 9))
    p = synth.small(f"rand{seed}", batch=batch, L=L, T=T, H=H, h=h, B=B, k=k, kprime=kprime,
                    dtype=dtype, needles=needles, seed=700 + seed)
    mmax = max(1, 8192 // B)
    m = int(rng.integers(1, min(mmax, 2 * p.M + 2) + 1))
    return p, m


# Number of seeded shapes (MISA_RANDOM_SHAPES / MISA_RANDOM_EXACT raise them
# for a longer sweep; MISA_RANDOM_FIRST / MISA_RANDOM_EXACT_FIRST start it
# at a later seed, so that a sweep can cover shapes not run before).
N_RANDOM = int(os.environ.get("MISA_RANDOM_SHAPES", "64"))
N_RANDOM_EXACT = int(os.environ.get("MISA_RANDOM_EXACT", "32"))
RANDOM_FIRST = int(os.environ.get("MISA_RANDOM_FIRST", "0"))
RANDOM_EXACT_FIRST = int(os.environ.get("MISA_RANDOM_EXACT_FIRST", "0"))


@pytest.mark.parametrize("seed", range(RANDOM_FIRST, RANDOM_FIRST + N_RANDOM))
def test_random_shapes(seed):
    p, m = _random_problem(seed)
    hisa = p.dtype != synth.F32
    x = synth.generate(p)
    neg = seed % 4 == 3  # signed weights: Eq. (9) keeps the sign (Eq. (7) takes |w|)
    if neg:
        sign = np.random.default_rng(3000 + seed).choice([-1.0, 1.0], size=tuple(x.w.shape))
        x.w.mul_(torch.from_numpy(sign).to(x.w.dtype))
    _log(f"[gpu] random shape {seed}: {p}" + (f", hisa m={m}" if hisa else "") + (", signed w" if neg else ""))
    stages = ("pool", "route", "score", "dense", "dagger", "step") + (("hisa",) if hisa else ())
    gpu = parity.run_gpu(x, stages=stages, m=m)
    op = parity.OracleProblem(x)
    tol = parity.TOL[p.dtype]
    qs = _all_queries(p)
    for b in range(p.batch):
        ref = op.seq(b).pooled
        np.testing.assert_allclose(gpu["pooled"][b], ref, rtol=1e-5, atol=1e-6 * np.abs(op.seq(b).K).max())
    parity.pmap(lambda bt: parity.check_query_misa(op, gpu, *bt, tol), qs)
    parity.pmap(lambda bt: parity.check_query_dense(op, gpu, *bt, tol), qs)
    if p.kprime:
        parity.pmap(lambda bt: parity.check_query_dagger(op, gpu, *bt, tol), qs)
    if "s_idx" in gpu:
        _check_step(op, gpu, qs, tol, f"rand{seed}")
    if hisa:
        parity.pmap(lambda bt: parity.check_query_hisa(op, gpu, *bt, tol), qs)


@pytest.mark.parametrize("seed", range(24))
def test_random_rerank_lists(seed):
    """misa_rerank on caller-made candidate lists: distinct prefix positions
    in random slots among -1 padding, some queries with fewer valid entries
    than k (or none), k' up to 8192, and row counts on both sides of the
    fused (one workgroup per query) and the separate list-select paths."""
    import long_context_pool_amd as misa

    rng = np.random.default_rng(8000 + seed)
    dtype = (synth.BF16, synth.FP8_E4M3)[seed % 2]
    H = int(rng.choice([16, 32, 64]))
    u = rng.random()
    T = 1 if u < 0.3 else (int(rng.integers(2, 9)) if u < 0.5 else int(rng.integers(100, 1301)))
    batch = int(rng.integers(1, 9)) if T <= 8 else 1
    L = int(rng.integers(T + 50, 9000))
    kprime = int(rng.integers(2, min(8192, L) + 1))
    k = int(rng.integers(1, kprime + 1))
    p = synth.small(f"rr{seed}", batch=batch, L=L, T=T, H=H, h=8, B=64, k=k, kprime=kprime,
                    dtype=dtype, needles=4, seed=600 + seed)
    x = synth.generate(p)
    cand = np.full((batch, T, kprime), -1, dtype=np.int32)
    for b in range(batch):
        for t in range(T):
            n = p.L - p.T + t + 1
            r = rng.random()
            nv = 0 if r < 0.03 else (int(rng.integers(1, min(n, k) + 1)) if r < 0.2 else int(rng.integers(1, min(n, kprime) + 1)))
            slots = rng.choice(kprime, size=nv, replace=False)
            cand[b, t, slots] = rng.choice(n, size=nv, replace=False)
    _log(f"[gpu] random rerank lists {seed}: {p}")
    dev = torch.device("cuda:0")
    fp8 = dtype == synth.FP8_E4M3
    q, kk, w = x.q.to(dev), x.k.to(dev), x.w.to(dev)
    qs = x.q_scale.to(dev) if fp8 else None
    ks = x.k_scale.to(dev) if fp8 else None
    shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
    ws = torch.empty(max(1, misa.misa_workspace_bytes(shp, p.h, k, kprime)), dtype=torch.uint8, device=dev)
    c = torch.from_numpy(cand).to(dev)
    idx = torch.empty((batch, T, k), dtype=torch.int32, device=dev)
    sc = torch.empty((batch, T, k), dtype=torch.float32, device=dev)
    misa.misa_rerank(shp, kprime, k, q, qs, w, kk, ks, c, idx, sc, ws)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    op = parity.OracleProblem(x)
    tol = parity.TOL[dtype]
    qs_all = _all_queries(p)
    if len(qs_all) > 48:  # the oracle re-scores k' candidates with every head: a spread sample
        pick = np.unique(np.linspace(0, len(qs_all) - 1, 48).astype(int))
        qs_all = [qs_all[i] for i in pick]
    parity.pmap(lambda bt: parity.check_rerank(op, cand[bt[0], bt[1]], idx[bt[0], bt[1]], sc[bt[0], bt[1]],
                                               bt[0], bt[1], tol), qs_all)


@pytest.mark.parametrize("seed", range(RANDOM_EXACT_FIRST, RANDOM_EXACT_FIRST + N_RANDOM_EXACT))
def test_random_shapes_exact(seed):
    """Random shapes on exact-integer inputs (every fp32 sum exact, heavy
    ties; now and then all keys from some position on the same row): every
    stage bit for bit, the oracle's tie rule included."""
    p, _ = _random_problem(1000 + seed)
    rng = np.random.default_rng(5000 + seed)
    p = dataclasses.replace(p, needles=0, kprime=p.kprime or min(p.k + 1 + int(rng.integers(0, p.k + 1)), 8192))
    x = synth.generate(p, exact_ints=True)
    if rng.random() < 0.3:
        dup = int(rng.integers(0, p.L))
        x.k[:, dup:] = x.k[:, dup:dup + 1].clone()
    neg = seed % 4 == 1
    if neg:  # signed weights (exact: +-2^-m)
        x.w.mul_(torch.from_numpy(rng.choice([-1.0, 1.0], size=tuple(x.w.shape))).to(x.w.dtype))
    _log(f"[gpu] random exact shape {seed}: {p}" + (", signed w" if neg else ""))
    gpu = parity.run_gpu(x)
    _check_exact(x, gpu)


# ---------------------------------------------------------------- exact arithmetic


def _check_exact(x, gpu):
    """Every stage of every query bit for bit against the oracle (given the
    GPU's own head set, which the router test checks within its tie band):
    the selected sets follow the oracle's tie rule exactly (lower token
    first) and the returned scores equal the oracle's as fp32."""
    import oracle

    p = x.problem
    op = parity.OracleProblem(x)

    def sel(what, got, ref):
        assert set(got.tolist()) == set(ref.tolist()), (
            f"{what}: {len(set(got.tolist()) ^ set(ref.tolist()))} indices differ")

    def vals(what, got_idx, got_sc, ref_scores):
        # Entries past a list shorter than k are padding: index -1, score -inf.
        v = got_idx >= 0
        assert np.all(got_sc[~v] == -np.inf), f"{what}: padding scores not -inf"
        np.testing.assert_array_equal(got_sc[v], ref_scores[got_idx[v]].astype(np.float32), err_msg=what)

    def one(bt):
        b, t = bt
        seq, pos, q, w = op.seq(b), op.pos(t), op.q[b, t], op.w[b, t]
        I = seq.scores(pos, q, w, gpu["heads"][b, t])
        sel(f"idx[{b},{t}]", gpu["idx"][b, t], oracle.topk(I, p.k))
        vals(f"scores[{b},{t}]", gpu["idx"][b, t], gpu["scores"][b, t], I)
        d = seq.dense(pos, q, w, p.k)
        sel(f"dense[{b},{t}]", gpu["d_idx"][b, t], d["idx"])
        vals(f"dense scores[{b},{t}]", gpu["d_idx"][b, t], gpu["d_scores"][b, t], d["scores"])
        sel(f"cand[{b},{t}]", gpu["cand"][b, t], oracle.topk(I, p.kprime))
        ridx, _ = oracle.rerank(seq.K, q, w, gpu["cand"][b, t], p.k)
        sel(f"rerank[{b},{t}]", gpu["r_idx"][b, t], ridx)
        if "s_idx" in gpu:
            Is = seq.scores(pos, q, w, gpu["s_heads"][b, t])
            sel(f"step idx[{b},{t}]", gpu["s_idx"][b, t], oracle.topk(Is, p.k))
            vals(f"step scores[{b},{t}]", gpu["s_idx"][b, t], gpu["s_scores"][b, t], Is)

    parity.pmap(one, _all_queries(p))


# name -> (batch, L, T, dup_from): T = 40 is the prefill path, T = 1 decode
# (batch 3: router partials + score kernels; batch 9: the single-kernel
# step), T = 4 multi-query decode.  dup_from: keys from that position on are
# all copies of one key, so thousands of scores tie bit for bit at the
# threshold digit: more than the decode select's 2048-entry list, which
# sends it to its full radix select.
EXACT = {
    "prefill_t40": (2, 1500, 40, None),
    "decode_b3": (3, 5000, 1, None),
    "decode_b9": (9, 3000, 1, None),
    "mq_t4": (2, 3000, 4, None),
    "decode_b3_mass_ties": (3, 8192, 1, 100),
    "decode_b9_mass_ties": (9, 8192, 1, 100),
    "mq_t4_mass_ties": (2, 8192, 4, 100),
}


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16, synth.FP8_E4M3])
@pytest.mark.parametrize("case", list(EXACT))
def test_exact_integer_inputs_bit_exact(case, dtype):
    """Small-integer q, k and power-of-two w: every fp32 partial sum is exact,
    so GPU scores equal the oracle's bit for bit and, with heavy ties, the
    selections must follow the oracle's rule exactly (lower index first)."""
    batch, L, T, dup_from = EXACT[case]
    if dtype == synth.F32 and T != 40:
        pytest.skip("fp32 inputs take the portable path, covered by the prefill case")
    p = synth.small(f"exact_{case}", batch=batch, L=L, T=T, H=64, h=8, B=64, k=200, kprime=400,
                    dtype=dtype, needles=0, seed=31)
    x = synth.generate(p, exact_ints=True)
    if dup_from is not None:
        x.k[:, dup_from:] = x.k[:, dup_from:dup_from + 1].clone()
    _log(f"[gpu] exact integers {case} {p}")
    gpu = parity.run_gpu(x)
    _check_exact(x, gpu)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8_E4M3])
def test_prefill_candidate_overflow_goes_to_repair(dtype):
    """Every key of a sequence the same row: all scores of a query tie, every
    key clears its split's threshold, and each (query, split) candidate
    segment overflows (four splits of 2048 keys against 640 or 768 slots).
    The writes past the capacity must stay inside their segment, and the
    repaired selections must be the oracle's: the lowest token indices."""
    import oracle

    p = synth.small("overflow", batch=2, L=8192, T=40, H=64, h=8, B=64, k=32, kprime=64,
                    dtype=dtype, needles=0, seed=50)
    x = synth.generate(p)
    x.k[:] = x.k[:, :1].clone()
    if dtype == synth.FP8_E4M3:
        x.k_scale[:] = x.k_scale[:, :1].clone()
    _log(f"[gpu] candidate overflow {p}")
    gpu = parity.run_gpu(x, stages=("pool", "route", "score", "dagger"))
    op = parity.OracleProblem(x)

    def one(bt):
        b, t = bt
        seq, pos = op.seq(b), op.pos(t)
        I = seq.scores(pos, op.q[b, t], op.w[b, t], gpu["heads"][b, t])
        for key, kk in (("idx", p.k), ("cand", p.kprime)):
            ref = oracle.topk(I, kk)
            assert set(gpu[key][b, t].tolist()) == set(ref.tolist()), f"{key}[{b},{t}]"
            assert set(ref.tolist()) == set(range(kk)), "all scores tie"

    parity.pmap(one, _all_queries(p))


def test_rerank_sequence_beyond_buffer_descriptor_reach():
    """Re-rank of a sequence whose keys span more than 2 GiB (bf16, L = 2^23 +
    2^16 keys of 256 bytes): such sequences are gathered with flat addresses
    (a buffer descriptor's offsets stop at 2 GiB).  Half of the candidates
    lie past the 2 GiB mark.  Exact-integer values: bit-exact against the
    oracle, which sees only the candidate rows (in token order, so its
    lower-index tie rule is the same)."""
    import torch

    import long_context_pool_amd as misa
    import oracle

    L, T, H, kp, k = (1 << 23) + (1 << 16), 2, 32, 512, 128
    p = synth.small("rerank_2gib", batch=1, L=L, T=T, H=H, h=8, B=128, k=k, kprime=kp,
                    dtype=synth.BF16, needles=0, seed=77)
    rng = np.random.Generator(np.random.PCG64(78))
    lo = rng.choice(1 << 23, size=kp // 2, replace=False)
    hi = (1 << 23) + rng.choice(L - T + 1 - (1 << 23), size=kp // 2, replace=False)
    rows = np.sort(np.concatenate([lo, hi]))
    x = synth.sparse_rows(p, rows)
    _log(f"[gpu] rerank beyond 2 GiB: L {L}, {kp} candidates, {kp // 2} past byte 2^31")
    dev = torch.device("cuda:0")
    shp = misa.shape(1, L, T, H, 128, p.B, p.dtype)
    q, kk, w = x.q.to(dev), x.k.to(dev), x.w.to(dev)
    cand_np = np.stack([rng.permutation(rows) for _ in range(T)]).astype(np.int32)[None]
    cand = torch.from_numpy(cand_np).to(dev)
    ws = torch.empty(misa.misa_workspace_bytes(shp, 8, k, kp), dtype=torch.uint8, device=dev)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    sc = torch.empty((1, T, k), dtype=torch.float32, device=dev)
    misa.misa_rerank(shp, kp, k, q, None, w, kk, None, cand, idx, sc, ws)
    torch.cuda.synchronize()
    gi, gs = idx.cpu().numpy()[0], sc.cpu().numpy()[0]
    Kc = oracle.decode(x.raw_numpy("k")[0][rows], oracle.BF16)
    qd = oracle.decode(x.raw_numpy("q")[0].reshape(T, -1), oracle.BF16).reshape(T, H, 128)
    for t in range(T):
        loc, ref_sc = oracle.rerank(Kc, qd[t], x.w[0, t].double().numpy(), np.arange(kp), k)
        assert set(gi[t].tolist()) == set(rows[loc].tolist()), f"rerank[{t}]"
        order = np.argsort(gi[t])
        ref = dict(zip(rows[loc].tolist(), ref_sc.tolist()))
        np.testing.assert_array_equal(gs[t][order],
                                      np.array([ref[i] for i in gi[t][order]], dtype=np.float32))
    del kk, q, ws
    torch.cuda.empty_cache()


def test_h_equals_H_matches_dense_on_gpu():
    p = synth.small("hH", batch=1, L=1000, T=20, H=16, h=16, B=64, k=100, kprime=None,
                    dtype=synth.BF16, needles=4, seed=32)
    x = synth.generate(p)
    gpu = parity.run_gpu(x, stages=("pool", "route", "score", "dense"))
    assert (gpu["heads"][0] == np.arange(16)).all()
    for t in range(p.T):
        assert set(gpu["idx"][0, t].tolist()) == set(gpu["d_idx"][0, t].tolist())


@pytest.mark.parametrize("dtype", [synth.BF16, synth.FP8_E4M3])
def test_negative_weights_decode_and_prefill(dtype):
    """Eq. (7) takes |w| for the router; Eq. (9) keeps the sign, so scores can
    be negative or -0.  Every other head's weight is negated."""
    for T in (1, 40):
        p = synth.small(f"negw_T{T}", batch=2, L=2600, T=T, H=64, h=8, B=64, k=300, kprime=None,
                        dtype=dtype, needles=8, seed=40 + T)
        x = synth.generate(p)
        x.w[..., ::2] *= -1.0
        _log(f"[gpu] negative weights {p}")
        gpu = parity.run_gpu(x, stages=("pool", "route", "score", "dense", "step"))
        op = parity.OracleProblem(x)
        tol = parity.TOL[p.dtype]
        qs = _all_queries(p)
        parity.pmap(lambda bt: parity.check_query_misa(op, gpu, *bt, tol), qs)
        parity.pmap(lambda bt: parity.check_query_dense(op, gpu, *bt, tol), qs)
        if "s_idx" in gpu:
            _check_step(op, gpu, qs, tol, p.name)


def test_repeat_runs_are_bit_identical():
    p = SMALL["bf16_ragged"]
    x = synth.generate(p)
    a = parity.run_gpu(x)
    b = parity.run_gpu(x)
    # Selections are sets: the slot order may differ, the (token, score) pairs may not.
    pairs = {"idx": "scores", "d_idx": "d_scores", "cand": "cand_scores", "r_idx": "r_scores"}
    for key, skey in pairs.items():
        oa, ob = np.argsort(a[key], axis=-1), np.argsort(b[key], axis=-1)
        np.testing.assert_array_equal(np.take_along_axis(a[key], oa, -1),
                                      np.take_along_axis(b[key], ob, -1), err_msg=key)
        np.testing.assert_array_equal(np.take_along_axis(a[skey], oa, -1),
                                      np.take_along_axis(b[skey], ob, -1), err_msg=skey)
    for key in ("pooled", "heads", "E"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_pool_range_updates_only_its_blocks():
    import torch

    import long_context_pool_amd as misa

    p = SMALL["bf16_ragged"]
    x = synth.generate(p)
    dev = torch.device("cuda:0")
    kk = x.k.to(dev)
    shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
    full = torch.empty((p.batch, p.M, p.d), dtype=torch.float32, device=dev)
    misa.misa_pool_keys(shp, kk, None, full)
    part = torch.full_like(full, 7.0)
    misa.misa_pool_keys_range(shp, p.M - 3, 3, kk, None, part)
    torch.cuda.synchronize()
    assert torch.equal(part[:, p.M - 3:], full[:, p.M - 3:])
    assert (part[:, :p.M - 3] == 7.0).all()


def test_status_codes_on_bad_arguments():
    import torch

    import long_context_pool_amd as misa

    dev = torch.device("cuda:0")
    shp = misa.shape(1, 256, 4, 64, 128, 64, misa.MISA_BF16)
    q = torch.zeros((1, 4, 64, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 256, 128), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((1, 4, 64), dtype=torch.float32, device=dev)
    heads = torch.zeros((1, 4, 8), dtype=torch.int32, device=dev)
    idx = torch.zeros((1, 4, 16), dtype=torch.int32, device=dev)
    ws_need = misa.misa_workspace_bytes(shp, 8, 16, 16)
    small_ws = torch.empty(max(16, ws_need // 2), dtype=torch.uint8, device=dev)
    with pytest.raises(misa.MisaError) as e:
        misa.misa_score_topk(shp, 8, 16, q, None, w, k, None, heads, idx, None, small_ws)
    assert e.value.status == misa.MISA_ERR_WORKSPACE
    ws = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    with pytest.raises(misa.MisaError) as e:
        misa.misa_score_topk(shp, 65, 16, q, None, w, k, None, heads, idx, None, ws)
    assert e.value.status == misa.MISA_ERR_INVALID_ARG
    with pytest.raises(misa.MisaError) as e:
        misa.misa_rerank(shp, 8, 16, q, None, w, k, None, idx, idx, None, ws)   # k' < k
    assert e.value.status == misa.MISA_ERR_INVALID_ARG
    bad = misa.shape(1, 256, 4, 64, 64, 64, misa.MISA_BF16)                      # d = 64
    with pytest.raises(misa.MisaError) as e:
        misa.dsa_index_dense(bad, 16, q, None, w, k, None, idx, None, ws)
    assert e.value.status == misa.MISA_ERR_UNSUPPORTED
    fp8 = misa.shape(1, 256, 4, 64, 128, 64, misa.MISA_FP8_E4M3)
    with pytest.raises(misa.MisaError) as e:                                      # no scales
        misa.dsa_index_dense(fp8, 16, q, None, w, k, None, idx, None, ws)
    assert e.value.status == misa.MISA_ERR_INVALID_ARG


def test_out_of_range_heads_and_candidates_are_ignored():
    """Caller-supplied head ids outside [0, H) contribute nothing, and
    candidates outside the query's prefix are skipped (no fault)."""
    import torch

    import long_context_pool_amd as misa
    import oracle

    p = synth.small("bad_ids", batch=1, L=600, T=8, H=64, h=8, B=64, k=32, kprime=64,
                    dtype=synth.BF16, needles=0, seed=33)
    x = synth.generate(p)
    op = parity.OracleProblem(x)
    dev = torch.device("cuda:0")
    q, kk, w = x.q.to(dev), x.k.to(dev), x.w.to(dev)
    shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
    ws = torch.empty(misa.misa_workspace_bytes(shp, p.h, p.k, p.kprime), dtype=torch.uint8, device=dev)
    heads = torch.tensor([[[0, 3, 5, 9, 64, 1000, -1, 7]] * p.T], dtype=torch.int32, device=dev)
    idx = torch.empty((1, p.T, p.k), dtype=torch.int32, device=dev)
    misa.misa_score_topk(shp, p.h, p.k, q, None, w, kk, None, heads, idx, None, ws)
    cand = torch.randint(0, p.L, (1, p.T, p.kprime), dtype=torch.int32)
    cand[..., :5] = torch.tensor([-1, p.L + 5, 2**31 - 1, -7, p.L - 1])
    ridx = torch.empty((1, p.T, p.k), dtype=torch.int32, device=dev)
    misa.misa_rerank(shp, p.kprime, p.k, q, None, w, kk, None, cand.to(dev), ridx, None, ws)
    torch.cuda.synchronize()
    for t in range(p.T):
        pos = op.pos(t)
        I = op.seq(0).scores(pos, op.q[0, t], op.w[0, t], np.array([0, 3, 5, 7, 9], np.int32))
        tau = parity.kth_value(I, p.k)
        parity.check_selection(idx.cpu().numpy()[0, t], oracle.topk(I, p.k), lambda s: I[s], tau,
                               1e-3, f"idx[{t}]")
        r = ridx.cpu().numpy()[0, t]
        assert all(0 <= s <= pos for s in r if s >= 0)


# ---------------------------------------------------------------- full-size workloads


def _tile_queries(p):
    """Decode: every sequence.  Prefill: one query of every 32-query workgroup
    tile, at a position inside the tile that walks through all 32 (so every
    row slot of the score kernel's A operand is checked somewhere)."""
    if p.T == 1:
        return [(b, 0) for b in range(p.batch)]
    tiles = (p.T + 31) // 32
    return [(0, min(p.T - 1, 32 * i + (i * 7) % 32)) for i in range(tiles)]


def _dense_queries(p, needles):
    """Dense DSA is 8x the routed work: every sequence in decode, else the
    first, second, middle and last query plus four needle targets."""
    if p.T == 1:
        return [(b, 0) for b in range(p.batch)]
    ts = sorted({0, 1, p.T // 2, p.T - 1} | {t for (_, _, t, _) in needles[:4]})
    return [(0, t) for t in ts]


FULL = ["c2", "c3", "c4", "c5"]
# Recall floors of the dense-DSA top-k on these synthetic workloads (measured
# 0.70 / 0.81 for MISA at C2 / C3 and 0.99 / 0.96 for MISA-dagger at C4 / C5):
# a gross error in any stage drops recall far below them.
RECALL_FLOOR = {"misa": 0.6, "dagger": 0.9}


@pytest.fixture(scope="module", params=FULL)
def full_case(request):
    p = synth.CONFIGS[request.param]
    _log(f"[gpu] full workload {request.param}: {p}")
    x = synth.generate(p)
    gpu = parity.run_gpu(x)
    return request.param, x, gpu, parity.OracleProblem(x)


def test_full_size_route_and_score(full_case):
    name, x, gpu, op = full_case
    p = x.problem
    tol = parity.TOL[p.dtype]
    qs = _tile_queries(p)
    res = parity.pmap(lambda bt: parity.check_query_misa(op, gpu, *bt, tol), qs)
    _log(f"[gpu] {name}: route + routed top-k ok on {len(qs)} queries; head swaps in band "
         f"{sum(r['head_swaps'] for r in res)}, token swaps in band {sum(r['tok_swaps'] for r in res)}")


def test_full_size_dense(full_case):
    name, x, gpu, op = full_case
    p = x.problem
    qs = _dense_queries(p, x.needles)
    res = parity.pmap(lambda bt: parity.check_query_dense(op, gpu, *bt, parity.TOL[p.dtype]), qs)
    _log(f"[gpu] {name}: dense ok on {len(qs)} queries; token swaps in band "
         f"{sum(r['dense_swaps'] for r in res)}")


def test_full_size_dagger(full_case):
    name, x, gpu, op = full_case
    p = x.problem
    if not p.kprime:
        pytest.skip("workload without MISA-dagger")
    qs = _tile_queries(p)
    res = parity.pmap(lambda bt: parity.check_query_dagger(op, gpu, *bt, parity.TOL[p.dtype]), qs)
    _log(f"[gpu] {name}: candidate pass + rerank ok on {len(qs)} queries; cand swaps "
         f"{sum(r['cand_swaps'] for r in res)}, rerank swaps {sum(r['rerank_swaps'] for r in res)}")


def test_full_size_decode_step(full_case):
    name, x, gpu, op = full_case
    p = x.problem
    if "s_idx" not in gpu:
        pytest.skip("misa_decode_step covers decode (T = 1)")
    _check_step(op, gpu, _tile_queries(p), parity.TOL[p.dtype], name)
    assert (gpu["s_idx"].min(axis=2) >= 0).all()


# MISA x HISA at the full workloads: m B = 8192 candidate tokens (4k).
HISA_FULL_M = {"c2": 128, "c3": 128, "c4": 64, "c5": 64}


def test_full_size_hisa(full_case):
    """The block scores, top-m blocks and the routed top-k inside them on the
    sampled queries, plus properties of every query's selection, and recall
    of the dense top-k against the MISA floor."""
    name, x, gpu, op = full_case
    p = x.problem
    m = HISA_FULL_M[name]
    hg = parity.run_gpu(x, stages=("pool", "route", "hisa"), m=m)
    qs = _tile_queries(p)
    res = parity.pmap(lambda bt: parity.check_query_hisa(op, hg, *bt, parity.TOL[p.dtype]), qs)
    pos = (p.L - p.T + np.arange(p.T))[None, :, None]
    a = hg["h_idx"]
    assert (a >= 0).all() and (a <= pos).all()
    assert (np.diff(np.sort(a, axis=2), axis=2) > 0).all(), "duplicate indices"
    for b in range(p.batch):
        for t0 in range(0, p.T, 256):
            blk = (a[b, t0:t0 + 256] // p.B)[..., None] == hg["hb"][b, t0:t0 + 256, None, :]
            assert blk.any(axis=2).all(), f"seq {b}: a token outside its query's blocks"
    rec = float(np.mean([len(np.intersect1d(a[i, t], gpu["d_idx"][i, t], assume_unique=True)) / p.k
                         for i in range(p.batch) for t in range(p.T)]))
    msg = (f"[gpu] {name}: MISA x HISA (m {m}) ok on {len(qs)} queries; block swaps "
           f"{sum(r['block_swaps'] for r in res)}, token swaps {sum(r['tok_swaps'] for r in res)}; "
           f"recall of dense top-k = {rec:.4f}")
    _log(msg)
    # On these inputs (i.i.d. keys, no block locality) block means say little,
    # so the floor is chance: m B of the L keys chosen at random (measured
    # 0.31 / 0.19 / 0.094 / 0.092 against 0.25 / 0.125 / 0.0625 / 0.0625 at
    # C2 / C3 / C4 / C5); a wrong block choice or scoring falls below it.
    assert rec >= m * p.B / p.L, msg


def test_full_size_output_properties_and_recall(full_case):
    """Whole-output properties that hold at any size (every query: indices in
    the causal prefix, distinct, no padding), and recall of the dense top-k."""
    name, x, gpu, op = full_case
    p = x.problem
    keys = ["idx", "d_idx"] + (["cand", "r_idx"] if p.kprime else [])
    pos = (p.L - p.T + np.arange(p.T))[None, :, None]
    for key in keys:
        a = gpu[key]
        assert (a >= 0).all() and (a <= pos).all(), key
        srt = np.sort(a, axis=2)
        assert (np.diff(srt, axis=2) > 0).all(), f"{key}: duplicate indices"
    if p.kprime:
        # Eq. (12): the re-ranked set is drawn from the query's own candidates.
        cs = np.sort(gpu["cand"], axis=2)
        for b in range(p.batch):
            for t in range(p.T):
                r = gpu["r_idx"][b, t]
                j = np.minimum(np.searchsorted(cs[b, t], r), cs.shape[2] - 1)
                assert (cs[b, t][j] == r).all(), f"rerank[{b},{t}]: index not a candidate"

    def recall(a, b):
        return float(np.mean([len(np.intersect1d(a[i, t], b[i, t], assume_unique=True)) / p.k
                              for i in range(p.batch) for t in range(p.T)]))

    rec = recall(gpu["idx"], gpu["d_idx"])
    msg = f"[gpu] {name}: MISA recall of dense top-k over all {p.batch * p.T} queries = {rec:.4f}"
    assert rec >= RECALL_FLOOR["misa"], msg
    if p.kprime:
        rec_d = recall(gpu["r_idx"], gpu["d_idx"])
        msg += f"; MISA-dagger recall = {rec_d:.4f}"
        assert rec_d >= RECALL_FLOOR["dagger"], msg
    _log(msg)


def test_decode_step_exchange_paths():
    """The single-kernel decode step (batch >= 8) shares router partials
    between the workgroups of a sequence once its workspace has been armed by
    a previous call; on a fresh (zeroed) workspace every workgroup computes
    the whole router itself.  Both paths add the same partials in the same
    order, so the two calls must agree bit for bit, and the second must match
    the oracle."""
    import torch

    import long_context_pool_amd as misa

    p = SMALL["bf16_decode_b8"]
    x = synth.generate(p)
    op = parity.OracleProblem(x)
    dev = torch.device("cuda:0")
    q, kk, w = x.q.to(dev), x.k.to(dev), x.w.to(dev)
    shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
    ws = torch.zeros(misa.misa_workspace_bytes(shp, p.h, p.k, p.k), dtype=torch.uint8, device=dev)
    pooled = torch.empty((p.batch, p.M, p.d), dtype=torch.float32, device=dev)
    misa.misa_pool_keys(shp, kk, None, pooled)
    runs = []
    for call in range(2):
        sp = pooled.clone()
        sp[:, p.M - 1].fill_(7.0)
        heads = torch.empty((p.batch, 1, p.h), dtype=torch.int32, device=dev)
        E = torch.empty((p.batch, 1, p.H), dtype=torch.float32, device=dev)
        idx = torch.empty((p.batch, 1, p.k), dtype=torch.int32, device=dev)
        sc = torch.empty((p.batch, 1, p.k), dtype=torch.float32, device=dev)
        misa.misa_decode_step(shp, p.h, p.k, q, None, w, sp, kk, None, heads, E, idx, sc, ws)
        torch.cuda.synchronize()
        runs.append({"s_pooled": sp.cpu().numpy(), "s_heads": heads.cpu().numpy(), "s_E": E.cpu().numpy(),
                     "s_idx": idx.cpu().numpy(), "s_scores": sc.cpu().numpy(), "pooled": pooled.cpu().numpy()})
    a, b = runs
    np.testing.assert_array_equal(a["s_E"].view(np.uint32), b["s_E"].view(np.uint32))
    np.testing.assert_array_equal(a["s_heads"], b["s_heads"])
    np.testing.assert_array_equal(a["s_pooled"], b["s_pooled"])
    for r in range(p.batch):
        oa, ob = np.argsort(a["s_idx"][r, 0]), np.argsort(b["s_idx"][r, 0])
        np.testing.assert_array_equal(a["s_idx"][r, 0][oa], b["s_idx"][r, 0][ob])
        np.testing.assert_array_equal(a["s_scores"][r, 0][oa].view(np.uint32), b["s_scores"][r, 0][ob].view(np.uint32))
    _check_step(op, b, _all_queries(p), parity.TOL[p.dtype], "exchange")
