"""GPU parity: every stage of the HIP path against the CPU oracle, through the
C ABI, on seeded synthetic inputs.

Small problems (several tiles, ragged tails, partial router blocks) are
checked on every query; the five full-size workloads on sampled queries
(first, last, middle, needle targets).  Tolerances and the tie-band rule are
in tests/parity.py.  Recall of the dense-DSA top-k is printed per problem.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

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
    "t_eq_l": synth.small("t_eq_l", batch=1, L=200, T=200, H=64, h=8, B=64, k=64, kprime=96,
                          dtype=synth.BF16, needles=0, seed=24),
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


# ---------------------------------------------------------------- exact arithmetic


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16, synth.FP8_E4M3])
def test_exact_integer_inputs_bit_exact(dtype):
    """Small-integer q, k and power-of-two w: every fp32 partial sum is exact,
    so GPU scores equal the oracle's bit for bit and, with heavy ties, the
    selections must follow the oracle's rule exactly (lower index first)."""
    import oracle

    p = synth.small("exact", batch=2, L=1500, T=40, H=64, h=8, B=64, k=200, kprime=400,
                    dtype=dtype, needles=0, seed=31)
    x = synth.generate(p, exact_ints=True)
    gpu = parity.run_gpu(x)
    op = parity.OracleProblem(x)

    def one(bt):
        b, t = bt
        seq, pos, q, w = op.seq(b), op.pos(t), op.q[b, t], op.w[b, t]
        heads = gpu["heads"][b, t]
        I = seq.scores(pos, q, w, heads)
        ref = oracle.topk(I, p.k)
        assert set(gpu["idx"][b, t].tolist()) == set(ref.tolist()), f"idx[{b},{t}]"
        np.testing.assert_array_equal(gpu["scores"][b, t], I[gpu["idx"][b, t]].astype(np.float32))
        d = seq.dense(pos, q, w, p.k)
        assert set(gpu["d_idx"][b, t].tolist()) == set(d["idx"].tolist()), f"dense[{b},{t}]"
        cref = oracle.topk(I, p.kprime)
        assert set(gpu["cand"][b, t].tolist()) == set(cref.tolist()), f"cand[{b},{t}]"
        ridx, rsc = oracle.rerank(seq.K, q, w, gpu["cand"][b, t], p.k)
        assert set(gpu["r_idx"][b, t].tolist()) == set(ridx.tolist()), f"rerank[{b},{t}]"

    parity.pmap(one, _all_queries(p))


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


def _sample_queries(p, needles):
    if p.T == 1:
        return [(b, 0) for b in range(min(p.batch, 6))]
    ts = sorted({0, 1, p.T // 2, p.T - 1} | {t for (_, _, t, _) in needles[:4]})
    return [(0, t) for t in ts]


FULL = ["c2", "c3", "c4", "c5"]


@pytest.fixture(scope="module", params=FULL)
def full_case(request):
    p = synth.CONFIGS[request.param]
    _log(f"[gpu] full workload {request.param}: {p}")
    x = synth.generate(p)
    gpu = parity.run_gpu(x)
    return request.param, x, gpu, parity.OracleProblem(x)


def test_full_size_sampled(full_case):
    name, x, gpu, op = full_case
    p = x.problem
    tol = parity.TOL[p.dtype]
    qs = _sample_queries(p, x.needles)
    res = parity.pmap(lambda bt: parity.check_query_misa(op, gpu, *bt, tol), qs)
    dres = parity.pmap(lambda bt: parity.check_query_dense(op, gpu, *bt, tol), qs)
    if p.kprime:
        parity.pmap(lambda bt: parity.check_query_dagger(op, gpu, *bt, tol), qs)
    # Whole-output properties that hold at any size.
    B_, T_, k_ = gpu["idx"].shape
    for b in range(B_):
        for t in range(T_):
            pos = op.pos(t)
            row = gpu["idx"][b, t]
            assert row.min() >= 0 and row.max() <= pos
            assert len(np.unique(row)) == k_
    if "s_idx" in gpu:
        _check_step(op, gpu, qs, tol, name)
        assert (gpu["s_idx"].min(axis=2) >= 0).all()
    rec = np.mean([len(set(gpu["idx"][b, t].tolist()) & set(gpu["d_idx"][b, t].tolist())) / p.k
                   for b in range(p.batch) for t in range(p.T)])
    _log(f"[gpu] {name}: sampled {len(qs)} queries ok; head swaps {sum(r['head_swaps'] for r in res)}, "
         f"MISA recall of dense top-k over all queries = {rec:.4f}")


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
