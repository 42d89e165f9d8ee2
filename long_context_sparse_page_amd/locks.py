"""ctypes binding of ``liblocks.so`` (C ABI in ``include/locks.h``).

Argument marshalling only: every function has the C name, takes device
tensors (or raw integer addresses), passes their pointers, and raises
``LocksError`` on a non-OK status.  Nothing here computes any part of the
decode path; if the library is missing the import fails loudly.
"""

from __future__ import annotations

import ctypes
import os

# The library must run on the same HIP runtime as torch (whose allocations and
# streams it is handed).  torch loads its own libamdhip64 (SONAME
# libamdhip64.so.7); importing torch first makes liblocks.so bind to that copy
# instead of loading a second runtime.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblocks.so")

LK_OK, LK_ERR_INVALID_ARG, LK_ERR_UNSUPPORTED, LK_ERR_WORKSPACE, LK_ERR_HIP = range(5)
LK_F32, LK_BF16 = 0, 1
LK_SUMMARY_KV, LK_SUMMARY_I4 = 0, 1

EXPORTED = (
    "lk_summary_record_bytes",
    "lk_page_budget",
    "lk_workspace_size",
    "lk_build_page_summary",
    "lk_score_select",
    "lk_sparse_decode_attn",
    "lk_dense_decode_attn",
    "lk_decode_step",
    "lk_decode_step_noalloc",
    "lk_status_string",
    "lk_last_error",
)


class LocksError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class lk_config(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("token_budget", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("summary_format", ctypes.c_int32),
    ]


class lk_cache(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("summary_pool", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m long_context_sparse_page_amd.build_lib`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfg, cache = ctypes.POINTER(lk_config), ctypes.POINTER(lk_cache)
    sig = {
        "lk_summary_record_bytes": (SZ, [cfg]),
        "lk_page_budget": (I32, [cfg]),
        "lk_workspace_size": (I32, [cfg, I32, I32, ctypes.POINTER(SZ)]),
        "lk_build_page_summary": (I32, [cfg, cache, P, I32, P, P, SZ, P]),
        "lk_score_select": (I32, [cfg, cache, I32, P, P, P, P, P, P, SZ, P]),
        "lk_sparse_decode_attn": (I32, [cfg, cache, I32, P, P, P, P, P, P, SZ, P]),
        "lk_dense_decode_attn": (I32, [cfg, cache, I32, P, P, P, P, SZ, P]),
        "lk_decode_step": (I32, [cfg, cache, I32, P, P, P, P, P, P, P, P, SZ, P]),
        "lk_decode_step_noalloc": (I32, [cfg, cache, I32, P, P, P, P, P, P, P, P]),
        "lk_status_string": (ctypes.c_char_p, [I32]),
        "lk_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != LK_OK:
        raise LocksError(status, _lib.lk_last_error().decode())


def make_config(head_dim=128, page_size=64, rank=8, num_q_heads=4, num_kv_heads=1,
                token_budget=512, kv_dtype=LK_F32, scale=None, summary_format=LK_SUMMARY_KV) -> lk_config:
    if scale is None:
        scale = head_dim ** -0.5
    return lk_config(head_dim, page_size, rank, num_q_heads, num_kv_heads, token_budget, kv_dtype, scale,
                     summary_format)


def make_cache(k_pool, v_pool, summary_pool, block_table, seq_lens) -> lk_cache:
    """Describe a cache from device tensors: pools [num_phys][Hkv][...],
    block_table int32 [batch][max_pages], seq_lens int32 [batch]."""
    n_phys = (k_pool if k_pool is not None else summary_pool).shape[0]
    return lk_cache(_ptr(k_pool), _ptr(v_pool), _ptr(summary_pool), _ptr(block_table),
                    _ptr(seq_lens), block_table.shape[1], n_phys)


def lk_summary_record_bytes(cfg: lk_config) -> int:
    return _lib.lk_summary_record_bytes(ctypes.byref(cfg))


def lk_page_budget(cfg: lk_config) -> int:
    return _lib.lk_page_budget(ctypes.byref(cfg))


def lk_workspace_size(cfg: lk_config, batch: int, max_pages_per_seq: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.lk_workspace_size(ctypes.byref(cfg), batch, max_pages_per_seq, ctypes.byref(out)))
    return out.value


def lk_build_page_summary(cfg, cache, phys_page_ids, n_pages, eigvals_out=None, ws=None,
                          ws_bytes=0, stream=None) -> None:
    _check(_lib.lk_build_page_summary(ctypes.byref(cfg), ctypes.byref(cache), _ptr(phys_page_ids),
                                      n_pages, _ptr(eigvals_out), _ptr(ws), ws_bytes, _stream(stream)))


def lk_score_select(cfg, cache, batch, q, page_lse_out, share_out, sel_pages, sel_count, ws,
                    ws_bytes, stream=None) -> None:
    _check(_lib.lk_score_select(ctypes.byref(cfg), ctypes.byref(cache), batch, _ptr(q), _ptr(page_lse_out),
                                _ptr(share_out), _ptr(sel_pages), _ptr(sel_count), _ptr(ws), ws_bytes,
                                _stream(stream)))


def lk_sparse_decode_attn(cfg, cache, batch, q, sel_pages, sel_count, out, lse_out, ws, ws_bytes,
                          stream=None) -> None:
    _check(_lib.lk_sparse_decode_attn(ctypes.byref(cfg), ctypes.byref(cache), batch, _ptr(q),
                                      _ptr(sel_pages), _ptr(sel_count), _ptr(out), _ptr(lse_out), _ptr(ws),
                                      ws_bytes, _stream(stream)))


def lk_dense_decode_attn(cfg, cache, batch, q, out, lse_out, ws, ws_bytes, stream=None) -> None:
    _check(_lib.lk_dense_decode_attn(ctypes.byref(cfg), ctypes.byref(cache), batch, _ptr(q), _ptr(out),
                                     _ptr(lse_out), _ptr(ws), ws_bytes, _stream(stream)))


def lk_decode_step(cfg, cache, batch, q, k_new, v_new, out, lse_out, sel_pages, sel_count, ws,
                   ws_bytes, stream=None) -> None:
    _check(_lib.lk_decode_step(ctypes.byref(cfg), ctypes.byref(cache), batch, _ptr(q), _ptr(k_new),
                               _ptr(v_new), _ptr(out), _ptr(lse_out), _ptr(sel_pages), _ptr(sel_count),
                               _ptr(ws), ws_bytes, _stream(stream)))


def lk_decode_step_noalloc(cfg, cache, batch, q, k_new, v_new, out, lse_out, sel_pages, sel_count,
                           stream=None) -> None:
    _check(_lib.lk_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(cache), batch, _ptr(q), _ptr(k_new),
                                       _ptr(v_new), _ptr(out), _ptr(lse_out), _ptr(sel_pages), _ptr(sel_count),
                                       _stream(stream)))


def lk_status_string(status: int) -> str:
    return _lib.lk_status_string(status).decode()


def lk_last_error() -> str:
    return _lib.lk_last_error().decode()
