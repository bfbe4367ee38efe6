"""CPU oracle for the MISA indexer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``long_context_pool_amd``) never imports it and it never imports the product.

The arithmetic lives in ``misa_oracle.cpp`` (plain single-threaded C++, double
precision, full sorts); this module builds it with g++, loads it with ctypes
and strings the per-equation functions together per query.  It follows the
MISA summary page ("MISA: Mixture of Indexer Sparse Attention for Long-Context
LLM Inference"): Eq. (1)-(2) in "Introduction and Theoretical Foundation",
Eq. (4), (7)-(10) in "Methodology" 1 and Eq. (11)-(12) in "Methodology" 2,
and the MISA x HISA combination that "Methodology" 1 ("Key distinction from
HISA") and "Theoretical and Practical Implications" ("Scalability") describe:
the Eq. (7) affinities reduced across heads to pick the top-m blocks.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, brute force, exact-arithmetic cases and the method's own
reductions (h = H gives DSA; k' >= n gives DSA).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "misa_oracle.cpp")
_LIB = os.path.join(_HERE, "_build", "libmisa_oracle.so")

# Element types of raw inputs (mirrors the C enum in misa_oracle.cpp).
F32, BF16, FP8_E4M3 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (no fast-math, no FMA contraction)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", "-o", tmp, _SRC,
        ])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.orc_decode.argtypes = [I32, P, P, I64, I64, P]
        lib.orc_pool.argtypes = [P, I64, I32, I32, P]
        lib.orc_expert_scores.argtypes = [P, P, I64, I32, I32, I32, P, P, P]
        lib.orc_top_heads.argtypes = [P, I32, I32, P]
        lib.orc_token_scores.argtypes = [P, I64, I32, P, P, P, I32, P]
        lib.orc_topk.argtypes = [P, I64, I32, P]
        lib.orc_rerank.argtypes = [P, I32, P, P, I32, P, I32, I32, P, P]
        lib.orc_block_scores.argtypes = [P, P, I64, I32, I32, I32, P, P, P]
        for f in (lib.orc_decode, lib.orc_pool, lib.orc_expert_scores, lib.orc_top_heads,
                  lib.orc_token_scores, lib.orc_topk, lib.orc_rerank, lib.orc_block_scores):
            f.restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- per-equation


def decode(raw: np.ndarray, dtype: int, row_scale: np.ndarray | None = None) -> np.ndarray:
    """Decode a raw [rows, cols] buffer (f32 / bf16 bits as uint16 / e4m3fn
    bytes as uint8) into float64; with ``row_scale`` row r is scaled by it."""
    raw = np.ascontiguousarray(raw)
    rows = raw.shape[0]
    cols = int(np.prod(raw.shape[1:])) if raw.ndim > 1 else 1
    out = np.empty((rows, cols), dtype=np.float64)
    sc = None if row_scale is None else _c(row_scale, np.float32)
    _load().orc_decode(dtype, _p(raw), None if sc is None else _p(sc), rows, cols, _p(out))
    return out.reshape(raw.shape)


def pool(K: np.ndarray, B: int) -> np.ndarray:
    """Eq. (4): mean of each block of B keys, K [L, d] -> [ceil(L/B), d]."""
    K = _c(K, np.float64)
    L, d = K.shape
    M = (L + B - 1) // B
    out = np.empty((M, d), dtype=np.float64)
    _load().orc_pool(_p(K), L, d, B, _p(out))
    return out


def expert_scores(K, pooled, pos: int, B: int, q_t, w_t) -> np.ndarray:
    """Eq. (7) for the query at position ``pos``: E [H]."""
    K = _c(K, np.float64)
    pooled = _c(pooled, np.float64)
    q_t = _c(q_t, np.float64)
    w_t = _c(w_t, np.float64)
    H, d = q_t.shape
    E = np.empty(H, dtype=np.float64)
    _load().orc_expert_scores(_p(K), _p(pooled), pos, d, B, H, _p(q_t), _p(w_t), _p(E))
    return E


def block_scores(K, pooled, pos: int, B: int, q_t, w_t) -> np.ndarray:
    """MISA x HISA block scores for the query at ``pos``: G [M_t], the Eq. (7)
    affinities summed over the heads."""
    K = _c(K, np.float64)
    pooled = _c(pooled, np.float64)
    q_t = _c(q_t, np.float64)
    w_t = _c(w_t, np.float64)
    H, d = q_t.shape
    G = np.empty((pos + 1 + B - 1) // B, dtype=np.float64)
    _load().orc_block_scores(_p(K), _p(pooled), pos, d, B, H, _p(q_t), _p(w_t), _p(G))
    return G


def top_heads(E, h: int) -> np.ndarray:
    """Eq. (8): the h heads with the largest E, ascending by head."""
    E = _c(E, np.float64)
    out = np.empty(h, dtype=np.int32)
    _load().orc_top_heads(_p(E), E.shape[0], h, _p(out))
    return out


def token_scores(K, pos: int, q_t, w_t, heads) -> np.ndarray:
    """Eq. (9) (Eq. (1) with all heads): scores of tokens 0..pos."""
    K = _c(K, np.float64)
    q_t = _c(q_t, np.float64)
    w_t = _c(w_t, np.float64)
    heads = _c(heads, np.int32)
    d = q_t.shape[1]
    out = np.empty(pos + 1, dtype=np.float64)
    _load().orc_token_scores(_p(K), pos, d, _p(q_t), _p(w_t), _p(heads), heads.shape[0], _p(out))
    return out


def topk(I, k: int) -> np.ndarray:
    """Eq. (2)/(10)/(11): indices of the k largest scores (rank order, -1 pad)."""
    I = _c(I, np.float64)
    out = np.empty(k, dtype=np.int32)
    _load().orc_topk(_p(I), I.shape[0], k, _p(out))
    return out


def rerank(K, q_t, w_t, cand, k: int):
    """Eq. (12): re-score the candidates with all heads, keep the k best.
    Returns (idx [k], Eq. (1) scores [k])."""
    K = _c(K, np.float64)
    q_t = _c(q_t, np.float64)
    w_t = _c(w_t, np.float64)
    cand = _c(cand, np.int32)
    H, d = q_t.shape
    idx = np.empty(k, dtype=np.int32)
    sc = np.empty(k, dtype=np.float64)
    _load().orc_rerank(_p(K), d, _p(q_t), _p(w_t), H, _p(cand), cand.shape[0], k, _p(idx), _p(sc))
    return idx, sc


# ---------------------------------------------------------------- per query


class Sequence:
    """One sequence's keys decoded to float64 plus its Eq. (4) pooled keys.

    ``K`` is [L, d] float64 (already dequantised); queries are addressed by
    absolute position ``pos`` (their causal prefix is keys 0..pos)."""

    def __init__(self, K: np.ndarray, B: int):
        self.K = _c(K, np.float64)
        self.B = B
        self.pooled = pool(self.K, B)

    def route(self, pos: int, q_t, w_t, h: int):
        """Eq. (7)-(8): (E [H], heads [h] ascending)."""
        E = expert_scores(self.K, self.pooled, pos, self.B, q_t, w_t)
        return E, top_heads(E, h)

    def scores(self, pos: int, q_t, w_t, heads) -> np.ndarray:
        return token_scores(self.K, pos, q_t, w_t, heads)

    def misa(self, pos: int, q_t, w_t, h: int, k: int):
        """Eq. (7)-(10) for one query: dict with E, heads, scores, idx."""
        E, heads = self.route(pos, q_t, w_t, h)
        I = self.scores(pos, q_t, w_t, heads)
        return {"E": E, "heads": heads, "scores": I, "idx": topk(I, k)}

    def dense(self, pos: int, q_t, w_t, k: int):
        """Eq. (1)-(2) for one query: dict with scores, idx."""
        H = np.asarray(q_t).shape[0]
        I = self.scores(pos, q_t, w_t, np.arange(H, dtype=np.int32))
        return {"scores": I, "idx": topk(I, k)}

    def block_scores(self, pos: int, q_t, w_t) -> np.ndarray:
        return block_scores(self.K, self.pooled, pos, self.B, q_t, w_t)

    def hisa_tokens(self, pos: int, q_t, w_t, heads, m: int, k: int):
        """MISA x HISA for one query: the top-m blocks by G (ties: lower
        block), then Eq. (9) with the given heads over the tokens of those
        blocks (causal: s <= pos) and the top-k of them (ties: lower token;
        -1 padding).  Returns dict with G, blocks (ascending), tokens (the
        candidate tokens, ascending), scores (Eq. (9) of each candidate) and
        idx (rank order)."""
        G = self.block_scores(pos, q_t, w_t)
        blocks = np.sort(topk(G, m))
        blocks = blocks[blocks >= 0]
        tokens = np.concatenate([np.arange(b * self.B, min((b + 1) * self.B, pos + 1))
                                 for b in blocks]).astype(np.int64)
        I = self.scores(pos, q_t, w_t, heads)
        cs = I[tokens]
        sel = topk(cs, k)
        idx = np.where(sel >= 0, tokens[np.maximum(sel, 0)], -1).astype(np.int32)
        return {"G": G, "blocks": blocks.astype(np.int32), "tokens": tokens, "scores": cs,
                "idx": idx}

    def misa_dagger(self, pos: int, q_t, w_t, h: int, kprime: int, k: int):
        """Eq. (11)-(12) for one query: dict with E, heads, cand, idx, scores."""
        r = self.misa(pos, q_t, w_t, h, kprime)
        idx, sc = rerank(self.K, q_t, w_t, r["idx"], k)
        return {"E": r["E"], "heads": r["heads"], "cand": r["idx"], "idx": idx, "scores": sc}
