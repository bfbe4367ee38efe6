"""Host-only checks of the C-ABI library: it loads, exports every entry point
that include/misa.h declares, and rejects bad arguments before launching
anything (these calls never reach the GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "misa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:misa|dsa)_[a-z_]+)\s*\(", text)))


def _param_counts():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for name, params in re.findall(r"\b((?:misa|dsa)_[a-z_]+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_lists_match_the_header():
    """Each ctypes signature has as many parameters as its C declaration (a
    missing one shifts the stream argument and crashes the launch)."""
    import long_context_pool_amd as misa

    lib = misa.lib()
    counts = _param_counts()
    assert set(counts) == set(_declared())
    for name, n in counts.items():
        assert len(getattr(lib, name).argtypes) == n, name


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("misa_pool_keys", "misa_route", "misa_score_topk", "misa_rerank", "dsa_index_dense",
              "misa_workspace_bytes", "misa_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import long_context_pool_amd as misa

    lib = ctypes.CDLL(misa.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(misa.EXPORTED) == set(_declared())


def test_status_strings():
    import long_context_pool_amd as misa

    assert misa.status_string(0) == "MISA_OK"
    assert misa.status_string(-3) == "MISA_ERR_WORKSPACE"


def test_workspace_bytes_zero_on_bad_shape():
    import long_context_pool_amd as misa

    assert misa.misa_workspace_bytes(misa.shape(1, 10, 20, 64, 128, 4, 1), 8, 4, 4) == 0  # T > L
    assert misa.misa_workspace_bytes(misa.shape(1, 100, 10, 64, 128, 4, 1), 8, 4, 4) > 0


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (calls fail validation)


@pytest.mark.parametrize("case,expect", [
    ("T>L", -1), ("d!=128", -2), ("h>H", -1), ("h>16", -2), ("k=0", -1), ("k>8192", -2),
    ("misaligned", -1), ("null q", -1), ("ws too small", -3), ("bad dtype", -1),
])
def test_argument_checks(case, expect):
    import long_context_pool_amd as misa

    lib = misa.lib()
    shp = misa.shape(1, 1024, 16, 64, 128, 64, misa.MISA_BF16)
    h, k, q, ws_bytes = 8, 32, FAKE, 1 << 40
    if case == "T>L":
        shp = misa.shape(1, 8, 16, 64, 128, 64, misa.MISA_BF16)
    elif case == "d!=128":
        shp = misa.shape(1, 1024, 16, 64, 64, 64, misa.MISA_BF16)
    elif case == "h>H":
        shp = misa.shape(1, 1024, 16, 8, 128, 64, misa.MISA_BF16)
        h = 9
    elif case == "h>16":
        h = 17
    elif case == "k=0":
        k = 0
    elif case == "k>8192":
        k = 8193
    elif case == "misaligned":
        q = FAKE + 4
    elif case == "null q":
        q = None
    elif case == "ws too small":
        ws_bytes = 16
    elif case == "bad dtype":
        shp = misa.shape(1, 1024, 16, 64, 128, 64, 7)
    st = lib.misa_score_topk(ctypes.byref(shp), h, k, q, None, FAKE, FAKE, None, FAKE, FAKE, None,
                             FAKE, ws_bytes, None)
    assert st == expect


def test_fp8_requires_scales_and_rerank_requires_kprime_ge_k():
    import long_context_pool_amd as misa

    lib = misa.lib()
    shp = misa.shape(1, 1024, 16, 64, 128, 64, misa.MISA_FP8_E4M3)
    st = lib.dsa_index_dense(ctypes.byref(shp), 32, FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE,
                             1 << 40, None)
    assert st == misa.MISA_ERR_INVALID_ARG
    shp = misa.shape(1, 1024, 16, 64, 128, 64, misa.MISA_BF16)
    st = lib.misa_rerank(ctypes.byref(shp), 16, 32, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None,
                         FAKE, 1 << 40, None)
    assert st == misa.MISA_ERR_INVALID_ARG
    st = lib.misa_pool_keys_range(ctypes.byref(shp), 10, 7, FAKE, None, FAKE, None)  # 17 > M=16
    assert st == misa.MISA_ERR_INVALID_ARG


@pytest.mark.parametrize("case,expect", [
    ("ok-shape, ws too small", -3), ("T=2", -2), ("fp32", -2), ("null pooled", -1),
    ("h>16", -2), ("fp8 without scales", -1),
])
def test_decode_step_argument_checks(case, expect):
    import long_context_pool_amd as misa

    lib = misa.lib()
    shp = misa.shape(4, 4096, 1, 64, 128, 64, misa.MISA_BF16)
    h, k, pooled, ws_bytes, qs = 8, 64, FAKE, 1 << 40, None
    if case == "ok-shape, ws too small":
        ws_bytes = misa.misa_workspace_bytes(shp, h, k, k) - 1
        assert ws_bytes > 0
    elif case == "T=2":
        shp = misa.shape(4, 4096, 2, 64, 128, 64, misa.MISA_BF16)
    elif case == "fp32":
        shp = misa.shape(4, 4096, 1, 64, 128, 64, misa.MISA_F32)
    elif case == "null pooled":
        pooled = None
    elif case == "h>16":
        h = 17
    elif case == "fp8 without scales":
        shp = misa.shape(4, 4096, 1, 64, 128, 64, misa.MISA_FP8_E4M3)
    st = lib.misa_decode_step(ctypes.byref(shp), h, k, FAKE, qs, FAKE, pooled, FAKE, None, FAKE,
                              None, FAKE, None, FAKE, ws_bytes, None)
    assert st == expect


@pytest.mark.parametrize("dtype", [1, 2])
def test_workspace_covers_both_selection_sizes(dtype):
    """misa_workspace_bytes(h, k, k') must cover misa_score_topk with k as
    well as with k'.  The prefill candidate capacity is not monotone in k: a
    k' large against L takes the lower sampling margin, so a k just below
    that point can need more than k'.  Shape of a 128K prefill (T 8192)."""
    import long_context_pool_amd as misa

    shp = misa.shape(1, 131072, 8192, 64, 128, 128, dtype)
    for k, kp in ((7000, 8192), (7900, 8192), (2048, 8192), (4000, 4096)):
        both = misa.misa_workspace_bytes(shp, 8, k, kp)
        assert both >= misa.misa_workspace_bytes(shp, 8, k, k), (k, kp)
        assert both >= misa.misa_workspace_bytes(shp, 8, kp, kp), (k, kp)


def test_noalloc_decode_step_rejects_shapes_beyond_its_scratch():
    """The no-allocation decode step refuses, before launching anything, a
    shape whose workspace exceeds its fixed scratch (batch 256 x L 2^20 needs
    about 1 GiB of scores), and applies misa_decode_step's argument checks."""
    import long_context_pool_amd as misa

    lib = misa.lib()
    big = misa.shape(256, 1 << 20, 1, 64, 128, 128, misa.MISA_BF16)
    st = lib.misa_decode_step_noalloc(ctypes.byref(big), 8, 64, FAKE, None, FAKE, FAKE, FAKE, None,
                                      FAKE, None, FAKE, None, None)
    assert st == misa.MISA_ERR_UNSUPPORTED
    shp = misa.shape(4, 4096, 2, 64, 128, 64, misa.MISA_BF16)  # T = 2
    st = lib.misa_decode_step_noalloc(ctypes.byref(shp), 8, 64, FAKE, None, FAKE, FAKE, FAKE, None,
                                      FAKE, None, FAKE, None, None)
    assert st == misa.MISA_ERR_UNSUPPORTED
    shp = misa.shape(4, 4096, 1, 64, 128, 64, misa.MISA_BF16)
    st = lib.misa_decode_step_noalloc(ctypes.byref(shp), 8, 64, FAKE, None, FAKE, None, FAKE, None,
                                      FAKE, None, FAKE, None, None)  # null pooled
    assert st == misa.MISA_ERR_INVALID_ARG
    assert misa.MISA_NOALLOC_SCRATCH_BYTES == 64 << 20


@pytest.mark.parametrize("case,expect", [
    ("ok-shape, ws too small", -3), ("fp32", -2), ("m=0", -1), ("m*B>8192", -2), ("h>16", -2),
    ("null heads", -1), ("null pooled", -1), ("k>8192", -2), ("misaligned blocks_out", -1),
])
def test_hisa_argument_checks(case, expect):
    import long_context_pool_amd as misa

    lib = misa.lib()
    shp = misa.shape(1, 4096, 64, 64, 128, 64, misa.MISA_BF16)
    h, m, k, pooled, heads, bo, ws_bytes = 8, 16, 256, FAKE, FAKE, None, 1 << 40
    if case == "ok-shape, ws too small":
        ws_bytes = misa.misa_hisa_workspace_bytes(shp, h, m, k) - 1
        assert ws_bytes > 0
    elif case == "fp32":
        shp = misa.shape(1, 4096, 64, 64, 128, 64, misa.MISA_F32)
    elif case == "m=0":
        m = 0
    elif case == "m*B>8192":
        m = 129
    elif case == "h>16":
        h = 17
    elif case == "null heads":
        heads = None
    elif case == "null pooled":
        pooled = None
    elif case == "k>8192":
        k = 8193
    elif case == "misaligned blocks_out":
        bo = FAKE + 4
    st = lib.misa_hisa_score_topk(ctypes.byref(shp), h, m, k, FAKE, None, FAKE, pooled, FAKE, None,
                                  heads, bo, None, FAKE, None, FAKE, ws_bytes, None)
    assert st == expect


def test_hisa_workspace_grows_with_the_candidate_list():
    """The HISA workspace holds m B candidates per query, or k when k is
    larger (the list is padded up to k)."""
    import long_context_pool_amd as misa

    shp = misa.shape(1, 65536, 4096, 64, 128, 64, misa.MISA_BF16)
    a = misa.misa_hisa_workspace_bytes(shp, 8, 32, 2048)   # 2048 candidates
    b = misa.misa_hisa_workspace_bytes(shp, 8, 128, 2048)  # 8192 candidates
    c = misa.misa_hisa_workspace_bytes(shp, 8, 8, 2048)    # 512 blocks' tokens, padded to 2048
    # c holds the same 2048 candidate scores per query as a, and 24 fewer
    # block slots per query.
    assert 0 < c < a < b
    assert a - c <= 4096 * 24 * 4 + 2 * 256
    assert misa.misa_hisa_workspace_bytes(shp, 8, 0, 2048) == 0
