"""misa_decode_step_noalloc (the decode step on the library's fixed device
scratch, for callers that cannot allocate) against misa_decode_step on a
caller workspace: two calls in a row through the C ABI, the second with a
smaller input, each compared bit for bit (the same kernels run on both
sides, so heads, E, the rebuilt pooled block and the selected (token, score)
pairs must be identical), and each checked against the CPU oracle."""

import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu

# Larger first, then smaller: the second call reuses the scratch left by the
# first (stale scores, histograms and router words of another shape).  Batch
# >= 8 runs the single-kernel step, batch < 8 the three-kernel form.
CALLS = [
    synth.small("noalloc_b9", batch=9, L=6000, T=1, H=64, h=8, B=64, k=300, kprime=None,
                dtype=synth.BF16, needles=8, seed=61),
    synth.small("noalloc_b3", batch=3, L=2500, T=1, H=32, h=8, B=128, k=200, kprime=None,
                dtype=synth.FP8_E4M3, needles=4, seed=62),
]


def _step(misa, fn, x, ws=None):
    import torch

    p = x.problem
    dev = torch.device("cuda:0")
    fp8 = p.dtype == synth.FP8_E4M3
    q, kk, w = x.q.to(dev), x.k.to(dev), x.w.to(dev)
    qs = x.q_scale.to(dev) if fp8 else None
    ks = x.k_scale.to(dev) if fp8 else None
    shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
    pooled = torch.empty((p.batch, p.M, p.d), dtype=torch.float32, device=dev)
    misa.misa_pool_keys(shp, kk, ks, pooled)
    pooled[:, p.M - 1].fill_(7.0)  # the step must rebuild the newest block
    heads = torch.empty((p.batch, 1, p.h), dtype=torch.int32, device=dev)
    E = torch.empty((p.batch, 1, p.H), dtype=torch.float32, device=dev)
    idx = torch.empty((p.batch, 1, p.k), dtype=torch.int32, device=dev)
    sc = torch.empty((p.batch, 1, p.k), dtype=torch.float32, device=dev)
    args = (shp, p.h, p.k, q, qs, w, pooled, kk, ks, heads, E, idx, sc)
    if ws is None:
        fn(*args)
    else:
        fn(*args, ws)
    torch.cuda.synchronize()
    return {"s_pooled": pooled.cpu().numpy(), "s_heads": heads.cpu().numpy(), "s_E": E.cpu().numpy(),
            "s_idx": idx.cpu().numpy(), "s_scores": sc.cpu().numpy()}


def test_noalloc_decode_step_matches_workspace_step():
    import torch

    import long_context_pool_amd as misa

    for p in CALLS:
        print(f"[gpu] no-alloc decode step {p}", flush=True)
        x = synth.generate(p)
        shp = misa.shape(p.batch, p.L, p.T, p.H, p.d, p.B, p.dtype)
        ws = torch.empty(misa.misa_workspace_bytes(shp, p.h, p.k, p.k), dtype=torch.uint8,
                         device="cuda:0")
        ref = _step(misa, misa.misa_decode_step, x, ws)
        got = _step(misa, misa.misa_decode_step_noalloc, x)
        np.testing.assert_array_equal(got["s_heads"], ref["s_heads"])
        np.testing.assert_array_equal(got["s_E"].view(np.uint32), ref["s_E"].view(np.uint32))
        np.testing.assert_array_equal(got["s_pooled"].view(np.uint32), ref["s_pooled"].view(np.uint32))
        for b in range(p.batch):
            og, orf = np.argsort(got["s_idx"][b, 0]), np.argsort(ref["s_idx"][b, 0])
            np.testing.assert_array_equal(got["s_idx"][b, 0][og], ref["s_idx"][b, 0][orf])
            np.testing.assert_array_equal(got["s_scores"][b, 0][og].view(np.uint32),
                                          ref["s_scores"][b, 0][orf].view(np.uint32))
        # And the oracle (route within its tie band, routed top-k given the
        # heads), as for misa_decode_step itself.
        op = parity.OracleProblem(x)
        view = {"E": got["s_E"], "heads": got["s_heads"], "idx": got["s_idx"], "scores": got["s_scores"]}
        qs = [(b, 0) for b in range(p.batch)]
        parity.pmap(lambda bt: parity.check_query_misa(op, view, *bt, parity.TOL[p.dtype]), qs)
        del ws
