"""Seeded synthetic inputs for the MISA indexer.

This module only draws random numbers and casts them; it holds none of the
indexer's arithmetic.  Both the GPU library's tests/benchmark and the CPU
oracle consume the exact bytes it produces.

Recipe (shapes and distributions of the MISA summary page's workloads:
DeepSeek-V3.2-like H=64 and GLM-5-like H=32 indexers, token budget k=2048,
needle-in-a-haystack style planted keys up to 128K context):

* per-head gain g_j = exp(N(0,1)), drawn once per problem;
* queries q[b,t,j,:] = g_j * N(0, I_d);
* keys k[b,s,:] ~ N(0, I_d);
* head weights w[b,t,j] = softplus(N(0,1)) / 8  (fp32, always positive);
* needles: ``needles`` distinct key positions per sequence, uniform in
  [0, L-T) (decode: [0, L-1)); each adds 3*q[b,t*,j*,:] to the key there,
  with the query t* and head j* uniform;
* casting: fp32 as drawn; bf16 by round-to-nearest-even; fp8 (OCP e4m3fn) with
  one fp32 scale per key token (amax over d / 448) and one per query token
  (amax over heads and d / 448), codes = saturating RNE of value / scale.

Queries of every sequence sit at positions L-T .. L-1.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

F32, BF16, FP8_E4M3 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8_E4M3: "fp8_e4m3"}
FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Problem:
    name: str
    batch: int
    L: int
    T: int
    H: int
    h: int
    d: int
    B: int
    k: int
    kprime: int | None
    dtype: int
    seed: int
    needles: int

    @property
    def M(self) -> int:
        return (self.L + self.B - 1) // self.B

    @property
    def pairs(self) -> int:
        """Scored (query, token) pairs: sum over queries of the causal prefix length."""
        per_seq = sum(self.L - self.T + t + 1 for t in range(self.T))
        return self.batch * per_seq


# The five workloads (tiny CPU-checkable, decode, prefill chunk, GLM-5 decode
# with MISA-dagger, 128K fp8 prefill with MISA-dagger).
C1 = Problem("tiny_fp32_L2048_T128", 1, 2048, 128, 64, 8, 128, 64, 256, None, F32, 1, 16)
C2 = Problem("decode_bf16_b32_L32768", 32, 32768, 1, 64, 8, 128, 64, 2048, None, BF16, 2, 64)
C3 = Problem("prefill_bf16_T4096_L65536", 1, 65536, 4096, 64, 8, 128, 64, 2048, None, BF16, 3, 64)
C4 = Problem("glm_decode_bf16_b8_L131072_dagger", 8, 131072, 1, 32, 8, 128, 128, 2048, 8192, BF16, 4, 64)
C5 = Problem("prefill_fp8_T8192_L131072_dagger", 1, 131072, 8192, 64, 8, 128, 128, 2048, 8192,
             FP8_E4M3, 5, 64)
CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


@dataclasses.dataclass
class Inputs:
    """Raw input buffers (host, contiguous).

    q: [batch, T, H, d], k: [batch, L, d] as torch tensors of float32,
    bfloat16 or float8_e4m3fn; q_scale [batch, T] and k_scale [batch, L] are
    float32 (all ones unless fp8); w [batch, T, H] float32.  ``needles`` is a
    list of (b, s, t, j) tuples."""

    problem: Problem
    q: torch.Tensor
    k: torch.Tensor
    w: torch.Tensor
    q_scale: torch.Tensor
    k_scale: torch.Tensor
    needles: list

    def raw_numpy(self, name: str) -> np.ndarray:
        """The tensor's bytes as numpy (uint16 for bf16, uint8 for fp8)."""
        t = getattr(self, name).contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.uint16).numpy()
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _to_fp8(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    y = (x / scale).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn)


def generate(p: Problem, seed: int | None = None, exact_ints: bool = False) -> Inputs:
    """Draw the inputs of problem ``p``.

    With ``exact_ints`` the values are small integers (q, k in [-4, 4]) and
    w = 2^-m (m in 0..3), which every input dtype holds exactly and whose
    scores are exact in fp32: used to force bit-identical scores and heavy
    ties.  Scales are then 1."""
    rng = np.random.Generator(np.random.PCG64(p.seed if seed is None else seed))
    b, L, T, H, d = p.batch, p.L, p.T, p.H, p.d
    if exact_ints:
        q = rng.integers(-4, 5, size=(b, T, H, d)).astype(np.float32)
        k = rng.integers(-4, 5, size=(b, L, d)).astype(np.float32)
        w = np.ldexp(1.0, -rng.integers(0, 4, size=(b, T, H))).astype(np.float32)
        needles = []
    else:
        gain = np.exp(rng.standard_normal(H)).astype(np.float32)
        q = rng.standard_normal((b, T, H, d), dtype=np.float32)
        q *= gain[None, None, :, None]
        k = rng.standard_normal((b, L, d), dtype=np.float32)
        w = (_softplus(rng.standard_normal((b, T, H))) / 8.0).astype(np.float32)
        needles = []
        span = max(L - T, 1)
        for bi in range(b):
            n = min(p.needles, span)
            pos = rng.choice(span, size=n, replace=False)
            tq = rng.integers(0, T, size=n)
            hq = rng.integers(0, H, size=n)
            for s, t, j in zip(pos.tolist(), tq.tolist(), hq.tolist()):
                k[bi, s] += 3.0 * q[bi, t, j]
                needles.append((bi, s, t, j))
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k)
    ones_q = torch.ones((b, T), dtype=torch.float32)
    ones_k = torch.ones((b, L), dtype=torch.float32)
    if p.dtype == F32:
        qr, kr, qs, ks = qt, kt, ones_q, ones_k
    elif p.dtype == BF16:
        qr, kr, qs, ks = qt.to(torch.bfloat16), kt.to(torch.bfloat16), ones_q, ones_k
    elif p.dtype == FP8_E4M3:
        if exact_ints:
            qs, ks = ones_q, ones_k
        else:
            qs = (qt.abs().amax(dim=(2, 3)) / FP8_MAX).clamp_min(1e-30)
            ks = (kt.abs().amax(dim=2) / FP8_MAX).clamp_min(1e-30)
        qr = _to_fp8(qt, qs[:, :, None, None])
        kr = _to_fp8(kt, ks[:, :, None])
    else:
        raise ValueError(f"unknown dtype {p.dtype}")
    return Inputs(p, qr.contiguous(), kr.contiguous(), torch.from_numpy(w).contiguous(),
                  qs.contiguous(), ks.contiguous(), needles)


def small(name: str, **kw) -> Problem:
    """A small problem for parity tests; unspecified fields follow C1."""
    base = dataclasses.asdict(C1)
    base.update(name=name, **kw)
    return Problem(**base)


def sparse_rows(p: Problem, rows: np.ndarray, seed: int | None = None) -> Inputs:
    """Exact-integer inputs (as ``generate(..., exact_ints=True)``) whose keys
    are zero except at the given key positions ``rows`` (the same for every
    sequence): a cheap stand-in for very long sequences where only a few
    rows are ever read.  Scales are 1.  Draw order: q, w, then the rows."""
    if p.dtype == F32:
        raise ValueError("sparse_rows holds bf16 or fp8 keys")
    rng = np.random.Generator(np.random.PCG64(p.seed if seed is None else seed))
    b, L, T, H, d = p.batch, p.L, p.T, p.H, p.d
    rows = np.asarray(rows, dtype=np.int64)
    q = rng.integers(-4, 5, size=(b, T, H, d)).astype(np.float32)
    w = np.ldexp(1.0, -rng.integers(0, 4, size=(b, T, H))).astype(np.float32)
    kv = rng.integers(-4, 5, size=(b, len(rows), d)).astype(np.float32)
    tdt = torch.bfloat16 if p.dtype == BF16 else torch.float8_e4m3fn
    k = torch.zeros((b, L, d), dtype=tdt)
    k[:, torch.from_numpy(rows)] = torch.from_numpy(kv).to(tdt)
    return Inputs(p, torch.from_numpy(q).to(tdt).contiguous(), k, torch.from_numpy(w).contiguous(),
                  torch.ones((b, T), dtype=torch.float32), torch.ones((b, L), dtype=torch.float32),
                  [])
