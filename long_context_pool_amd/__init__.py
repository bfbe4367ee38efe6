"""Python binding of the MISA indexer C ABI (``include/misa.h``).

Argument marshalling only: every function has the C entry point's name and
arguments, takes device tensors (torch) or raw device addresses (int), passes
their addresses and sizes to ``libmisa.so`` and raises :class:`MisaError` on a
non-OK status.  All computation happens in the library's HIP kernels; there is
no CPU fallback -- importing this package fails if the library is not built.

MISA (Mixture of Indexer Sparse Attention) is the drop-in replacement for the
DeepSeek Sparse Attention token indexer described on the MISA summary page
("MISA: Mixture of Indexer Sparse Attention for Long-Context LLM Inference").
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmisa.so")

MISA_OK = 0
MISA_ERR_INVALID_ARG = -1
MISA_ERR_UNSUPPORTED = -2
MISA_ERR_WORKSPACE = -3
MISA_ERR_HIP = -4

MISA_F32, MISA_BF16, MISA_FP8_E4M3 = 0, 1, 2

EXPORTED = (
    "misa_workspace_bytes", "misa_pool_keys", "misa_pool_keys_range", "misa_route",
    "misa_score_topk", "misa_decode_step", "misa_decode_step_noalloc", "misa_rerank",
    "dsa_index_dense", "misa_hisa_workspace_bytes", "misa_hisa_score_topk", "misa_status_string",
)
MISA_NOALLOC_SCRATCH_BYTES = 64 << 20


class MisaError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


class misa_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "L", "T", "H", "d", "B", "qk_dtype")]


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m long_context_pool_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_SHP = ctypes.POINTER(misa_shape)

_lib.misa_workspace_bytes.argtypes = [_SHP, _I32, _I32, _I32]
_lib.misa_workspace_bytes.restype = _SZ
_lib.misa_pool_keys.argtypes = [_SHP, _P, _P, _P, _P]
_lib.misa_pool_keys_range.argtypes = [_SHP, _I32, _I32, _P, _P, _P, _P]
_lib.misa_route.argtypes = [_SHP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.misa_score_topk.argtypes = [_SHP, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.misa_decode_step.argtypes = [_SHP, _I32, _I32] + [_P] * 11 + [_SZ, _P]
_lib.misa_decode_step_noalloc.argtypes = [_SHP, _I32, _I32] + [_P] * 11
_lib.misa_hisa_workspace_bytes.argtypes = [_SHP, _I32, _I32, _I32]
_lib.misa_hisa_workspace_bytes.restype = _SZ
_lib.misa_hisa_score_topk.argtypes = [_SHP, _I32, _I32, _I32] + [_P] * 12 + [_SZ, _P]
_lib.misa_rerank.argtypes = [_SHP, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.dsa_index_dense.argtypes = [_SHP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
for _f in ("misa_pool_keys", "misa_pool_keys_range", "misa_route", "misa_score_topk",
           "misa_decode_step", "misa_decode_step_noalloc", "misa_rerank", "dsa_index_dense",
           "misa_hisa_score_topk"):
    getattr(_lib, _f).restype = ctypes.c_int
_lib.misa_status_string.argtypes = [ctypes.c_int]
_lib.misa_status_string.restype = ctypes.c_char_p


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.misa_status_string(status).decode()


def shape(batch, L, T, H, d, B, qk_dtype) -> misa_shape:
    return misa_shape(batch, L, T, H, d, B, qk_dtype)


def _ptr(x):
    """Device address of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws) -> int:
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def _check(status: int, fn: str):
    if status != MISA_OK:
        raise MisaError(status, fn)


def misa_workspace_bytes(shp: misa_shape, h: int, k: int, kprime: int) -> int:
    return int(_lib.misa_workspace_bytes(ctypes.byref(shp), h, k, kprime))


def misa_pool_keys(shp, k, k_scale, pooled, stream=None):
    _check(_lib.misa_pool_keys(ctypes.byref(shp), _ptr(k), _ptr(k_scale), _ptr(pooled),
                               _stream(stream)), "misa_pool_keys")


def misa_pool_keys_range(shp, block_begin, block_count, k, k_scale, pooled, stream=None):
    _check(_lib.misa_pool_keys_range(ctypes.byref(shp), block_begin, block_count, _ptr(k),
                                     _ptr(k_scale), _ptr(pooled), _stream(stream)),
           "misa_pool_keys_range")


def misa_route(shp, h, q, q_scale, w, pooled, k, k_scale, heads, E_out, ws, stream=None):
    _check(_lib.misa_route(ctypes.byref(shp), h, _ptr(q), _ptr(q_scale), _ptr(w), _ptr(pooled),
                           _ptr(k), _ptr(k_scale), _ptr(heads), _ptr(E_out), _ptr(ws),
                           _nbytes(ws), _stream(stream)), "misa_route")


def misa_score_topk(shp, h, k, q, q_scale, w, kk, k_scale, heads, idx, scores_out, ws,
                    stream=None):
    _check(_lib.misa_score_topk(ctypes.byref(shp), h, k, _ptr(q), _ptr(q_scale), _ptr(w),
                                _ptr(kk), _ptr(k_scale), _ptr(heads), _ptr(idx),
                                _ptr(scores_out), _ptr(ws), _nbytes(ws), _stream(stream)),
           "misa_score_topk")


def misa_decode_step(shp, h, k, q, q_scale, w, pooled, kk, k_scale, heads, E_out, idx,
                     scores_out, ws, stream=None):
    _check(_lib.misa_decode_step(ctypes.byref(shp), h, k, _ptr(q), _ptr(q_scale), _ptr(w),
                                 _ptr(pooled), _ptr(kk), _ptr(k_scale), _ptr(heads), _ptr(E_out),
                                 _ptr(idx), _ptr(scores_out), _ptr(ws), _nbytes(ws),
                                 _stream(stream)), "misa_decode_step")


def misa_decode_step_noalloc(shp, h, k, q, q_scale, w, pooled, kk, k_scale, heads, E_out, idx,
                             scores_out, stream=None):
    _check(_lib.misa_decode_step_noalloc(ctypes.byref(shp), h, k, _ptr(q), _ptr(q_scale), _ptr(w),
                                         _ptr(pooled), _ptr(kk), _ptr(k_scale), _ptr(heads),
                                         _ptr(E_out), _ptr(idx), _ptr(scores_out),
                                         _stream(stream)), "misa_decode_step_noalloc")


def misa_rerank(shp, kprime, k, q, q_scale, w, kk, k_scale, cand, idx, scores_out, ws,
                stream=None):
    _check(_lib.misa_rerank(ctypes.byref(shp), kprime, k, _ptr(q), _ptr(q_scale), _ptr(w),
                            _ptr(kk), _ptr(k_scale), _ptr(cand), _ptr(idx), _ptr(scores_out),
                            _ptr(ws), _nbytes(ws), _stream(stream)), "misa_rerank")


def dsa_index_dense(shp, k, q, q_scale, w, kk, k_scale, idx, scores_out, ws, stream=None):
    _check(_lib.dsa_index_dense(ctypes.byref(shp), k, _ptr(q), _ptr(q_scale), _ptr(w), _ptr(kk),
                                _ptr(k_scale), _ptr(idx), _ptr(scores_out), _ptr(ws),
                                _nbytes(ws), _stream(stream)), "dsa_index_dense")


def misa_hisa_workspace_bytes(shp: misa_shape, h: int, m: int, k: int) -> int:
    return int(_lib.misa_hisa_workspace_bytes(ctypes.byref(shp), h, m, k))


def misa_hisa_score_topk(shp, h, m, k, q, q_scale, w, pooled, kk, k_scale, heads, blocks_out,
                         block_scores_out, idx, scores_out, ws, stream=None):
    _check(_lib.misa_hisa_score_topk(ctypes.byref(shp), h, m, k, _ptr(q), _ptr(q_scale), _ptr(w),
                                     _ptr(pooled), _ptr(kk), _ptr(k_scale), _ptr(heads),
                                     _ptr(blocks_out), _ptr(block_scores_out), _ptr(idx),
                                     _ptr(scores_out), _ptr(ws), _nbytes(ws), _stream(stream)),
           "misa_hisa_score_topk")
