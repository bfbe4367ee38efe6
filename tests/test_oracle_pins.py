"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the MISA summary page and plain
mathematics fix: a hand-worked example (tests/golden), closed forms, brute
force on tiny inputs, numpy float64 library routines (an independent
implementation), exact-arithmetic inputs, and the method's own reductions
(h = H is DSA; k' >= n is DSA; k' = k is MISA).  A plausible slip anywhere in
the oracle -- a dropped partial block, ReLU on the wrong side, an off-by-one
prefix, a transposed operand, a wrong tie rule -- fails at least one test.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


# ------------------------------------------------------------ hand example


def test_hand_example():
    g = json.load(open(GOLDEN))
    K = np.array(g["K"], dtype=np.float64)
    seq = oracle.Sequence(K, g["B"])
    np.testing.assert_array_equal(seq.pooled, np.array(g["pooled"], dtype=np.float64))
    for qd in g["queries"]:
        q = np.array(qd["q"], dtype=np.float64)
        w = np.array(qd["w"], dtype=np.float64)
        E, heads = seq.route(qd["pos"], q, w, qd["h"])
        np.testing.assert_allclose(E, qd["E"], rtol=1e-15, atol=0)
        assert heads.tolist() == qd["heads"]
        I = seq.scores(qd["pos"], q, w, heads)
        assert I.tolist() == qd["routed_scores"]
        if "routed_top4" in qd:
            assert oracle.topk(I, 4).tolist() == qd["routed_top4"]
            d = seq.dense(qd["pos"], q, w, 3)
            assert d["scores"].tolist() == qd["dense_scores"]
            assert d["idx"].tolist() == qd["dense_top3"]
            r = seq.misa_dagger(qd["pos"], q, w, qd["h"], qd["dagger_kprime"], qd["dagger_k"])
            assert r["cand"].tolist() == qd["dagger_cand"]
            assert r["idx"].tolist() == qd["dagger_idx"]
            assert r["scores"].tolist() == qd["dagger_scores"]
        else:
            assert oracle.topk(I, 2).tolist() == qd["routed_top2"]


# ------------------------------------------------------------ decoding


def test_decode_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    ours = oracle.decode(codes, oracle.BF16)
    ref = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_decode_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    ours = oracle.decode(codes, oracle.FP8_E4M3)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    # Named points of the OCP E4M3 format.
    flat = ours.reshape(-1)
    assert flat[0x38] == 1.0 and flat[0x7E] == 448.0 and flat[0x01] == 2.0 ** -9
    assert np.isnan(flat[0x7F]) and np.isnan(flat[0xFF])
    assert flat[0xB8] == -1.0


def test_decode_row_scale():
    codes = np.array([[0x38, 0x40], [0x38, 0xC0]], dtype=np.uint8)  # 1, 2 / 1, -2
    out = oracle.decode(codes, oracle.FP8_E4M3, np.array([0.5, 3.0], dtype=np.float32))
    np.testing.assert_array_equal(out, [[0.5, 1.0], [3.0, -6.0]])


# ------------------------------------------------------------ Eq. (4) pool


def test_pool_constant_block_and_partial_mean():
    rng = np.random.default_rng(0)
    L, d, B = 37, 5, 8
    K = rng.standard_normal((L, d))
    P = oracle.pool(K, B)
    assert P.shape == (5, d)
    for b in range(5):
        np.testing.assert_allclose(P[b], K[b * B:min(b * B + B, L)].mean(axis=0), rtol=1e-13)
    Kc = np.repeat(rng.standard_normal((1, d)), L, axis=0)
    np.testing.assert_allclose(oracle.pool(Kc, B), np.repeat(Kc[:1], 5, axis=0), rtol=1e-14)


def test_pool_is_linear():
    rng = np.random.default_rng(1)
    K1, K2 = rng.standard_normal((20, 4)), rng.standard_normal((20, 4))
    np.testing.assert_allclose(oracle.pool(2.0 * K1 - 3.0 * K2, 6),
                               2.0 * oracle.pool(K1, 6) - 3.0 * oracle.pool(K2, 6), rtol=1e-12, atol=1e-14)


def test_pool_B1_is_identity():
    K = np.random.default_rng(2).standard_normal((9, 3))
    np.testing.assert_array_equal(oracle.pool(K, 1), K)


# ------------------------------------------------------------ Eq. (7) E


def _numpy_E(K, pos, B, q, w):
    """Independent float64 numpy statement of Eq. (7) with the causal prefix."""
    n = pos + 1
    blocks = [K[b:min(b + B, n)].mean(axis=0) for b in range(0, n, B)]
    Kb = np.stack(blocks)                                  # [M_t, d]
    A = w[:, None] * np.maximum(q @ Kb.T, 0.0)             # [H, M_t]
    return np.abs(A).mean(axis=1)


@pytest.mark.parametrize("pos", [0, 5, 63, 64, 65, 130, 199])
def test_expert_scores_match_numpy(pos):
    rng = np.random.default_rng(3)
    L, d, H, B = 200, 16, 6, 64
    K = rng.standard_normal((L, d))
    q = rng.standard_normal((H, d)) * np.exp(rng.standard_normal(H))[:, None]
    w = np.abs(rng.standard_normal(H))
    seq = oracle.Sequence(K, B)
    E, _ = seq.route(pos, q, w, 2)
    np.testing.assert_allclose(E, _numpy_E(K, pos, B, q, w), rtol=1e-12, atol=1e-300)


def test_expert_scores_negative_weight_uses_abs():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((40, 8))
    q = rng.standard_normal((3, 8))
    w = np.array([-0.7, 0.3, -2.0])
    seq = oracle.Sequence(K, 16)
    E, _ = seq.route(39, q, w, 1)
    np.testing.assert_allclose(E, _numpy_E(K, 39, 16, q, w), rtol=1e-12)
    assert (E >= 0).all()
    E_abs, _ = seq.route(39, q, np.abs(w), 1)
    np.testing.assert_array_equal(E, E_abs)


def test_expert_scores_special_cases_B1_and_single_block():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((12, 4))
    q = rng.standard_normal((3, 4))
    w = np.array([0.5, 1.0, 2.0])
    # B = 1: pooled keys are the keys themselves; E_j = |w_j| * mean_s ReLU(q_j.k_s).
    E, _ = oracle.Sequence(K, 1).route(7, q, w, 1)
    np.testing.assert_allclose(E, w * np.maximum(q @ K[:8].T, 0).mean(axis=1), rtol=1e-13)
    # One block covering the whole prefix (n <= B): E_j = |w_j| ReLU(q_j.mean(k_0..k_pos)).
    E, _ = oracle.Sequence(K, 16).route(7, q, w, 1)
    np.testing.assert_allclose(E, w * np.maximum(q @ K[:8].mean(axis=0), 0), rtol=1e-13)


# ------------------------------------------------------------ Eq. (8), (2)/(10) top-k


def _brute_topk(v, k):
    order = sorted(range(len(v)), key=lambda i: (-v[i], i))
    return [order[r] if r < len(v) else -1 for r in range(k)]


@pytest.mark.parametrize("seed", range(5))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    v = rng.integers(0, 6, size=50).astype(np.float64)  # heavy ties
    for k in (1, 7, 50, 60):
        got = oracle.topk(v, k)
        assert got.tolist() == _brute_topk(v.tolist(), k)
        sel = got[got >= 0]
        assert len(sel) == min(k, 50)
        if k < 50:
            rest = np.setdiff1d(np.arange(50), sel)
            assert v[sel].min() >= v[rest].max()


@pytest.mark.parametrize("seed", range(5))
def test_top_heads_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    E = rng.integers(0, 4, size=16).astype(np.float64)
    for h in (1, 4, 8, 16):
        got = oracle.top_heads(E, h)
        assert got.tolist() == sorted(_brute_topk(E.tolist(), h))


# ------------------------------------------------------------ Eq. (9), (1) scores


def test_token_scores_match_numpy():
    rng = np.random.default_rng(6)
    L, d, H = 300, 32, 8
    K = rng.standard_normal((L, d))
    q = rng.standard_normal((H, d))
    w = np.abs(rng.standard_normal(H))
    heads = np.array([1, 4, 6], dtype=np.int32)
    pos = 211
    I = oracle.token_scores(K, pos, q, w, heads)
    ref = (w[heads, None] * np.maximum(q[heads] @ K[:pos + 1].T, 0.0)).sum(axis=0)
    np.testing.assert_allclose(I, ref, rtol=1e-12, atol=1e-12)


def test_exact_integer_inputs_are_bit_exact():
    """Small-integer q, k and power-of-two w: every partial sum is exact, so the
    oracle must agree bit-for-bit with numpy (float64) and with float32."""
    p = synth.small("exact", L=256, T=16, H=8, h=2, d=32, B=16, k=32)
    x = synth.generate(p, exact_ints=True)
    K = x.k[0].double().numpy()
    q = x.q[0].double().numpy()
    w = x.w[0].double().numpy()
    seq = oracle.Sequence(K, p.B)
    for t in (0, 7, 15):
        pos = p.L - p.T + t
        I = seq.scores(pos, q[t], w[t], np.arange(p.H, dtype=np.int32))
        ref64 = (w[t][:, None] * np.maximum(q[t] @ K[:pos + 1].T, 0)).sum(axis=0)
        qf, kf, wf = q[t].astype(np.float32), K[:pos + 1].astype(np.float32), w[t].astype(np.float32)
        ref32 = (wf[:, None] * np.maximum(qf @ kf.T, 0)).sum(axis=0, dtype=np.float32)
        np.testing.assert_array_equal(I, ref64)
        np.testing.assert_array_equal(I, ref32.astype(np.float64))


# ------------------------------------------------------------ method reductions


def _small_problem_seq(seed=7, L=512, T=24, H=16, d=32, B=32):
    p = synth.small("red", L=L, T=T, H=H, h=4, d=d, B=B, k=40, needles=4, seed=seed)
    x = synth.generate(p)
    return p, oracle.Sequence(x.k[0].double().numpy(), B), x.q[0].double().numpy(), x.w[0].double().numpy()


def test_h_equals_H_is_dense_bit_exact():
    p, seq, q, w = _small_problem_seq()
    for t in range(0, p.T, 5):
        pos = p.L - p.T + t
        m = seq.misa(pos, q[t], w[t], p.H, p.k)
        d = seq.dense(pos, q[t], w[t], p.k)
        np.testing.assert_array_equal(m["scores"], d["scores"])
        np.testing.assert_array_equal(m["idx"], d["idx"])


def test_dagger_with_kprime_ge_n_is_dense():
    p, seq, q, w = _small_problem_seq(L=200, T=8)
    for t in range(p.T):
        pos = p.L - p.T + t
        r = seq.misa_dagger(pos, q[t], w[t], 4, pos + 1 + 3, p.k)   # k' > n: padded candidates
        d = seq.dense(pos, q[t], w[t], p.k)
        np.testing.assert_array_equal(r["idx"], d["idx"])
        np.testing.assert_array_equal(r["scores"], d["scores"][d["idx"]])


def test_dagger_with_kprime_eq_k_keeps_the_misa_set():
    p, seq, q, w = _small_problem_seq()
    for t in range(0, p.T, 3):
        pos = p.L - p.T + t
        r = seq.misa_dagger(pos, q[t], w[t], 4, p.k, p.k)
        m = seq.misa(pos, q[t], w[t], 4, p.k)
        assert set(r["idx"].tolist()) == set(m["idx"].tolist())


def test_dagger_recall_identity_and_monotone_in_kprime():
    """Eq. (12) keeps the k best of Omega under the dense score, so it holds every
    dense-top-k token that lies in Omega: |T_dagger & T_dsa| = |T_dsa & Omega|,
    and a larger k' (a superset Omega) can only raise it."""
    p, seq, q, w = _small_problem_seq()
    for t in range(0, p.T, 4):
        pos = p.L - p.T + t
        dense = set(seq.dense(pos, q[t], w[t], p.k)["idx"].tolist())
        prev = -1
        for kp in (p.k, 2 * p.k, 4 * p.k):
            r = seq.misa_dagger(pos, q[t], w[t], 4, kp, p.k)
            omega = set(r["cand"].tolist())
            hit = len(set(r["idx"].tolist()) & dense)
            assert hit == len(dense & omega)
            assert hit >= prev
            prev = hit


def test_causality_future_keys_do_not_matter():
    p, seq, q, w = _small_problem_seq()
    t = 5
    pos = p.L - p.T + t
    a = seq.misa(pos, q[t], w[t], 4, p.k)
    K2 = seq.K.copy()
    K2[pos + 1:] = np.random.default_rng(99).standard_normal(K2[pos + 1:].shape) * 50
    b = oracle.Sequence(K2, p.B).misa(pos, q[t], w[t], 4, p.k)
    np.testing.assert_array_equal(a["E"], b["E"])
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["scores"], b["scores"])


def test_prefill_query_equals_decode_call_on_its_prefix():
    p, seq, q, w = _small_problem_seq()
    t = 9
    pos = p.L - p.T + t
    a = seq.misa(pos, q[t], w[t], 4, p.k)
    short = oracle.Sequence(seq.K[:pos + 1], p.B)
    b = short.misa(pos, q[t], w[t], 4, p.k)
    np.testing.assert_allclose(a["E"], b["E"], rtol=1e-14)
    np.testing.assert_array_equal(a["idx"], b["idx"])


def test_own_position_is_in_the_prefix():
    p, seq, q, w = _small_problem_seq()
    t = 3
    pos = p.L - p.T + t
    K2 = seq.K.copy()
    K2[pos] = 20.0 * q[t].sum(axis=0)          # a key every head scores highly
    r = oracle.Sequence(K2, p.B).dense(pos, q[t], w[t], 1)
    assert r["idx"][0] == pos
    assert len(oracle.Sequence(K2, p.B).scores(pos, q[t], w[t], [0])) == pos + 1


def test_positive_scaling_and_head_permutation():
    p, seq, q, w = _small_problem_seq()
    t = 11
    pos = p.L - p.T + t
    a = seq.misa(pos, q[t], w[t], 4, p.k)
    b = seq.misa(pos, q[t], 4.0 * w[t], 4, p.k)        # power of two: exact
    np.testing.assert_array_equal(a["heads"], b["heads"])
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(4.0 * a["scores"], b["scores"])
    perm = np.random.default_rng(3).permutation(p.H)
    c = seq.misa(pos, q[t][perm], w[t][perm], 4, p.k)
    np.testing.assert_allclose(c["E"], a["E"][perm], rtol=1e-14)
    assert sorted(perm[c["heads"]].tolist()) == a["heads"].tolist()
    assert set(c["idx"].tolist()) == set(a["idx"].tolist())


def test_short_prefix_pads_with_minus_one():
    p, seq, q, w = _small_problem_seq(L=30, T=30, B=8)
    r = seq.misa(4, q[4], w[4], 4, 10)        # n = 5 < k = 10
    assert sorted(r["idx"][:5].tolist()) == [0, 1, 2, 3, 4]
    assert r["idx"][5:].tolist() == [-1] * 5


# ------------------------------------------------------------ MISA x HISA


def test_hisa_hand_example():
    g = json.load(open(GOLDEN))
    seq = oracle.Sequence(np.array(g["K"], dtype=np.float64), g["B"])
    for qd in g["queries"]:
        q = np.array(qd["q"], dtype=np.float64)
        w = np.array(qd["w"], dtype=np.float64)
        G = seq.block_scores(qd["pos"], q, w)
        assert G.tolist() == qd["hisa_G"]
        for case in qd["hisa_cases"]:
            r = seq.hisa_tokens(qd["pos"], q, w, np.array(qd["heads"], np.int32), case["m"], case["k"])
            assert r["blocks"].tolist() == case["blocks"], case
            assert r["idx"].tolist() == case["idx"], case


def test_hisa_block_scores_with_B1_are_the_dense_token_scores():
    """B = 1: every pooled key is its token's key and no block is partial, so
    G_b is Eq. (1) of token b (summed by a different oracle routine)."""
    p = synth.small("hisa_b1", L=300, T=3, B=1, dtype=synth.F32, needles=2, seed=61)
    x = synth.generate(p)
    K = x.k[0].double().numpy()
    seq = oracle.Sequence(K, 1)
    for t in range(p.T):
        pos = p.L - p.T + t
        q, w = x.q[0, t].double().numpy(), x.w[0, t].double().numpy()
        G = seq.block_scores(pos, q, w)
        I = seq.scores(pos, q, w, np.arange(p.H, dtype=np.int32))
        np.testing.assert_array_equal(G, I)


@pytest.mark.parametrize("pos", [511, 517, 700])
def test_hisa_single_head_block_scores_give_the_expert_score(pos):
    """H = 1: G_b is that head's A_b, so Eq. (7)'s E = mean_b |G_b| (complete
    and partial blocks alike)."""
    p = synth.small("hisa_h1", L=701, T=1, H=1, h=1, B=64, dtype=synth.F32, needles=0, seed=62)
    x = synth.generate(p)
    seq = oracle.Sequence(x.k[0].double().numpy(), p.B)
    q, w = x.q[0, 0].double().numpy(), x.w[0, 0].double().numpy()
    w = -w  # the sign survives in G, not in E
    G = seq.block_scores(pos, q, w)
    assert len(G) == (pos + 1 + p.B - 1) // p.B
    E, _ = seq.route(pos, q, w, 1)
    np.testing.assert_allclose(E[0], np.abs(G).mean(), rtol=1e-14)
    assert (G <= 0).all()


def test_hisa_with_every_block_is_misa():
    """m >= M_t keeps every token of the prefix, so the restricted top-k is
    the plain Eq. (10) top-k, and with every head it is Eq. (2)."""
    p = synth.small("hisa_all", L=900, T=4, B=64, k=50, dtype=synth.BF16, needles=4, seed=63)
    x = synth.generate(p)
    K = oracle.decode(x.raw_numpy("k")[0], oracle.BF16)
    seq = oracle.Sequence(K, p.B)
    qd = oracle.decode(x.raw_numpy("q")[0].reshape(p.T, -1), oracle.BF16).reshape(p.T, p.H, p.d)
    for t in range(p.T):
        pos = p.L - p.T + t
        w = x.w[0, t].double().numpy()
        E, heads = seq.route(pos, qd[t], w, p.h)
        r = seq.hisa_tokens(pos, qd[t], w, heads, 64, p.k)
        assert r["tokens"].tolist() == list(range(pos + 1))
        assert r["idx"].tolist() == seq.misa(pos, qd[t], w, p.h, p.k)["idx"].tolist()
        rd = seq.hisa_tokens(pos, qd[t], w, np.arange(p.H, dtype=np.int32), 64, p.k)
        assert rd["idx"].tolist() == seq.dense(pos, qd[t], w, p.k)["idx"].tolist()


def test_hisa_causality_and_planted_block():
    """Keys after the query change nothing; a block whose keys all lie along
    the scored heads' query directions (every dot product large and
    positive, all w > 0) is selected, and its tokens lead the top-k."""
    p = synth.small("hisa_plant", L=1024, T=1, B=64, dtype=synth.F32, needles=0, seed=64)
    x = synth.generate(p)
    K = x.k[0].double().numpy().copy()
    q, w = x.q[0, 0].double().numpy(), x.w[0, 0].double().numpy()
    pos = 700
    heads = np.arange(8, dtype=np.int32)
    base = oracle.Sequence(K, p.B).hisa_tokens(pos, q, w, heads, 3, 20)
    K2 = K.copy()
    K2[pos + 1:] = 100.0
    fut = oracle.Sequence(K2, p.B).hisa_tokens(pos, q, w, heads, 3, 20)
    assert fut["blocks"].tolist() == base["blocks"].tolist() and fut["idx"].tolist() == base["idx"].tolist()
    np.testing.assert_array_equal(fut["G"], base["G"])
    K3 = K.copy()
    K3[5 * 64:6 * 64] = 100.0 * sum(q[j] / np.linalg.norm(q[j]) for j in heads)
    r = oracle.Sequence(K3, p.B).hisa_tokens(pos, q, w, heads, 3, 20)
    assert 5 in r["blocks"].tolist()
    assert np.argmax(r["G"]) == 5
    assert set(r["idx"].tolist()) <= set(range(5 * 64, 6 * 64))
