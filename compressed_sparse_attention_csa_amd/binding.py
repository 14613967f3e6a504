"""Thin ctypes binding of libcsa.so (the C ABI in include/csa.h).

Argument marshalling only: torch tensors become device pointers, Python ints
become host int32 arrays, and the current torch stream is passed as the HIP
stream. Every step of the computation runs in the library's HIP kernels.
Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

CSA_MAX_LAYERS = 8
CSA_PAGE_ENTRIES = 64
CSA_HEAD_DIM = 128
CSA_IDX_DIM = 64
CSA_MAX_TOPK = 2048
CSA_POOL_BLOCK = 8
CSA_MAX_POOL_BLOCKS = 2048

CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_FP4_E2M1 = 0, 1, 2, 3
DTYPE_CODES = {"f32": CSA_F32, "bf16": CSA_BF16, "fp8": CSA_FP8_E4M3, "fp4": CSA_FP4_E2M1}

STATUS = {0: "CSA_OK", 1: "CSA_ERR_INVALID_ARG", 2: "CSA_ERR_SHAPE", 3: "CSA_ERR_DTYPE",
          4: "CSA_ERR_CAPACITY", 5: "CSA_ERR_UNSUPPORTED", 6: "CSA_ERR_HIP"}

ERR_PAGE, ERR_TOPK, ERR_FALLBACK = 1, 2, 4


class CsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "ratio", "head_dim", "q_heads", "idx_heads", "idx_dim", "window", "ring_rows", "n_layers",
        "max_seqs", "max_pages_per_seq", "pool_pages", "kv_dtype", "act_dtype", "swa_dtype")]


class Buffers(C.Structure):
    _fields_ = [
        ("kbar", C.c_void_p * CSA_MAX_LAYERS),
        ("vbar", C.c_void_p * CSA_MAX_LAYERS),
        ("kbar_scale", C.c_void_p * CSA_MAX_LAYERS),
        ("vbar_scale", C.c_void_p * CSA_MAX_LAYERS),
        ("kbar_stage", C.c_void_p * CSA_MAX_LAYERS),
        ("vbar_stage", C.c_void_p * CSA_MAX_LAYERS),
        ("kbar_gscale", C.c_void_p * CSA_MAX_LAYERS),
        ("vbar_gscale", C.c_void_p * CSA_MAX_LAYERS),
        ("ring_k", C.c_void_p * CSA_MAX_LAYERS),
        ("ring_v", C.c_void_p * CSA_MAX_LAYERS),
        ("ring_k_scale", C.c_void_p * CSA_MAX_LAYERS),
        ("ring_v_scale", C.c_void_p * CSA_MAX_LAYERS),
        ("block_stage", C.c_void_p * CSA_MAX_LAYERS),
        ("kidx", C.c_void_p),
        ("kidx_scale", C.c_void_p),
        ("kidx_stage", C.c_void_p),
        ("block_table", C.c_void_p),
        ("workspace", C.c_void_p),
        ("workspace_bytes", C.c_size_t),
    ]


class BufferSizes(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in (
        "kv_pool", "idx_pool", "page_scale", "kv_stage", "idx_stage", "group_scale", "ring", "ring_scale",
        "block_stage", "block_table")]


EXPORTS = [
    "csa_status_string", "csa_last_error", "csa_buffer_sizes_for", "csa_workspace_size",
    "csa_cache_create", "csa_cache_destroy", "csa_seq_reset", "csa_seq_len", "csa_seq_set_len",
    "csa_compress", "csa_index_topk", "csa_attend", "csa_read_errors",
    "csa_profile_begin", "csa_profile_end", "csa_debug_convert", "csa_attend_dense",
    "csa_seq_set_swa_start", "csa_ring_write", "csa_index_topk_pool", "csa_index_reindex",
    "csa_debug_stream_read", "csa_attend_noalloc",
]

_LIB = None


def lib() -> C.CDLL:
    """Load libcsa.so (once). Raises if it is missing: there is no fallback path."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m compressed_sparse_attention_csa_amd.csrc.build`")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    pi32 = C.POINTER(C.c_int32)
    L.csa_status_string.restype = C.c_char_p
    L.csa_status_string.argtypes = [C.c_int]
    L.csa_last_error.restype = C.c_char_p
    L.csa_last_error.argtypes = []
    L.csa_buffer_sizes_for.restype = C.c_int
    L.csa_buffer_sizes_for.argtypes = [C.POINTER(Config), C.POINTER(BufferSizes)]
    L.csa_workspace_size.restype = sz
    L.csa_workspace_size.argtypes = [C.POINTER(Config), i32, i32]
    L.csa_cache_create.restype = C.c_int
    L.csa_cache_create.argtypes = [C.POINTER(Config), C.POINTER(Buffers), C.POINTER(vp)]
    L.csa_cache_destroy.restype = C.c_int
    L.csa_cache_destroy.argtypes = [vp]
    L.csa_seq_reset.restype = C.c_int
    L.csa_seq_reset.argtypes = [vp, i32]
    L.csa_seq_len.restype = i64
    L.csa_seq_len.argtypes = [vp, i32, i32]
    L.csa_seq_set_len.restype = C.c_int
    L.csa_seq_set_len.argtypes = [vp, i32, i32, i64]
    L.csa_compress.restype = C.c_int
    L.csa_compress.argtypes = [vp, i32, i32, pi32, pi32, vp, vp, vp, vp, vp]
    L.csa_index_topk.restype = C.c_int
    L.csa_index_topk.argtypes = [vp, i32, pi32, pi32, vp, vp, i32, vp, vp]
    L.csa_index_topk_pool.restype = C.c_int
    L.csa_index_topk_pool.argtypes = [vp, i32, pi32, pi32, vp, vp, i32, vp, i32, vp, vp]
    L.csa_index_reindex.restype = C.c_int
    L.csa_index_reindex.argtypes = [vp, i32, pi32, pi32, vp, vp, i32, vp, i32, vp, vp]
    L.csa_attend.restype = C.c_int
    L.csa_attend.argtypes = [vp, i32, i32, pi32, pi32, vp, vp, i32, C.c_float, vp, vp]
    L.csa_attend_noalloc.restype = C.c_int
    L.csa_attend_noalloc.argtypes = [vp, i32, i32, pi32, pi32, vp, vp, i32, C.c_float, vp, vp]
    L.csa_attend_dense.restype = C.c_int
    L.csa_attend_dense.argtypes = [vp, i32, i32, pi32, pi32, vp, C.c_float, vp, vp]
    L.csa_seq_set_swa_start.restype = C.c_int
    L.csa_seq_set_swa_start.argtypes = [vp, i32, i32]
    L.csa_ring_write.restype = C.c_int
    L.csa_ring_write.argtypes = [vp, i32, i32, pi32, pi32, pi32, vp, vp, vp]
    L.csa_read_errors.restype = C.c_int
    L.csa_read_errors.argtypes = [vp, vp, C.POINTER(C.c_uint32)]
    L.csa_profile_begin.restype = C.c_int
    L.csa_profile_begin.argtypes = [vp, C.c_int32]
    L.csa_profile_end.restype = C.c_int
    L.csa_profile_end.argtypes = [vp, C.c_int32, C.POINTER(C.c_double), pi32]
    L.csa_debug_convert.restype = C.c_int
    L.csa_debug_convert.argtypes = [i32, vp, vp, i64, vp]
    L.csa_debug_stream_read.restype = C.c_int
    L.csa_debug_stream_read.argtypes = [C.POINTER(C.c_void_p), i32, i64, i32, vp, C.POINTER(C.c_float)]
    _LIB = L
    return L


def check(status: int) -> None:
    if status != 0:
        raise CsaError(status, lib().csa_last_error().decode())


def _i32(values) -> C.Array:
    vals = [int(v) for v in values]
    return (C.c_int32 * max(1, len(vals)))(*vals)


def _ptr(t: torch.Tensor | None):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# --------------------------------------------------------------------------- host-only calls

def csa_buffer_sizes_for(cfg: Config) -> BufferSizes:
    out = BufferSizes()
    check(lib().csa_buffer_sizes_for(C.byref(cfg), C.byref(out)))
    return out


def csa_workspace_size(cfg: Config, max_queries: int, max_k: int) -> int:
    return int(lib().csa_workspace_size(C.byref(cfg), max_queries, max_k))


def csa_cache_create(cfg: Config, bufs: Buffers) -> int:
    h = C.c_void_p()
    check(lib().csa_cache_create(C.byref(cfg), C.byref(bufs), C.byref(h)))
    return h.value


def csa_cache_destroy(h: int) -> None:
    check(lib().csa_cache_destroy(C.c_void_p(h)))


def csa_seq_reset(h: int, seq: int) -> None:
    check(lib().csa_seq_reset(C.c_void_p(h), seq))


def csa_seq_len(h: int, layer: int, seq: int) -> int:
    return int(lib().csa_seq_len(C.c_void_p(h), layer, seq))


def csa_seq_set_len(h: int, layer: int, seq: int, length: int) -> None:
    check(lib().csa_seq_set_len(C.c_void_p(h), layer, seq, length))


def csa_seq_set_swa_start(h: int, seq: int, start: int) -> None:
    check(lib().csa_seq_set_swa_start(C.c_void_p(h), seq, start))


# --------------------------------------------------------------------------- device calls

def csa_ring_write(h: int, layer: int, seq_ids, pos0, n_rows, raw_k, raw_v, stream=None) -> None:
    check(lib().csa_ring_write(C.c_void_p(h), layer, len(seq_ids), _i32(seq_ids), _i32(pos0), _i32(n_rows),
                               _ptr(raw_k), _ptr(raw_v), _stream(stream)))


def csa_compress(h: int, layer: int, seq_ids, n_new, raw_k, raw_v, gate, proj_idx=None, stream=None) -> None:
    check(lib().csa_compress(C.c_void_p(h), layer, len(seq_ids), _i32(seq_ids), _i32(n_new),
                             _ptr(raw_k), _ptr(raw_v), _ptr(gate), _ptr(proj_idx), _stream(stream)))


def csa_index_topk(h: int, q_seq, q_pos, q_idx, w_idx, k: int, topk, stream=None) -> None:
    check(lib().csa_index_topk(C.c_void_p(h), len(q_seq), _i32(q_seq), _i32(q_pos), _ptr(q_idx), _ptr(w_idx),
                               k, _ptr(topk), _stream(stream)))


def csa_index_topk_pool(h: int, q_seq, q_pos, q_idx, w_idx, k: int, topk, n_pool_blocks: int, pool,
                        stream=None) -> None:
    check(lib().csa_index_topk_pool(C.c_void_p(h), len(q_seq), _i32(q_seq), _i32(q_pos), _ptr(q_idx), _ptr(w_idx),
                                    k, _ptr(topk), n_pool_blocks, _ptr(pool), _stream(stream)))


def csa_index_reindex(h: int, q_seq, q_pos, q_idx, w_idx, n_pool_blocks: int, pool, k: int, topk,
                      stream=None) -> None:
    check(lib().csa_index_reindex(C.c_void_p(h), len(q_seq), _i32(q_seq), _i32(q_pos), _ptr(q_idx), _ptr(w_idx),
                                  n_pool_blocks, _ptr(pool), k, _ptr(topk), _stream(stream)))


def csa_attend(h: int, layer: int, q_seq, q_pos, q, topk, k: int, scale: float, out, stream=None) -> None:
    check(lib().csa_attend(C.c_void_p(h), layer, len(q_seq), _i32(q_seq), _i32(q_pos), _ptr(q), _ptr(topk),
                           k, float(scale), _ptr(out), _stream(stream)))


def csa_attend_noalloc(h: int, layer: int, q_seq, q_pos, q, topk, k: int, scale: float, out, stream=None) -> None:
    check(lib().csa_attend_noalloc(C.c_void_p(h), layer, len(q_seq), _i32(q_seq), _i32(q_pos), _ptr(q), _ptr(topk),
                                   k, float(scale), _ptr(out), _stream(stream)))


def csa_attend_dense(h: int, layer: int, q_seq, q_pos, q, scale: float, out, stream=None) -> None:
    check(lib().csa_attend_dense(C.c_void_p(h), layer, len(q_seq), _i32(q_seq), _i32(q_pos), _ptr(q),
                                 float(scale), _ptr(out), _stream(stream)))


def csa_read_errors(h: int, stream=None) -> int:
    v = C.c_uint32(0)
    check(lib().csa_read_errors(C.c_void_p(h), _stream(stream), C.byref(v)))
    return int(v.value)


PROFILE_INDEX = 1    # CSA_PROFILE_INDEX
PROFILE_ATTEND = 2   # CSA_PROFILE_ATTEND


def csa_profile_begin(h: int, kernels: int = PROFILE_INDEX) -> None:
    check(lib().csa_profile_begin(C.c_void_p(h), int(kernels)))


def csa_profile_end(h: int, kernel: int = PROFILE_INDEX) -> tuple[float, int]:
    ms = C.c_double(0.0)
    n = C.c_int32(0)
    check(lib().csa_profile_end(C.c_void_p(h), int(kernel), C.byref(ms), C.byref(n)))
    return float(ms.value), int(n.value)


def csa_debug_convert(kind: int, inp: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    check(lib().csa_debug_convert(kind, _ptr(inp), _ptr(out), inp.numel(), _stream(stream)))


def csa_debug_stream_read(bufs, nbytes: int, reps: int, stream=None) -> float:
    """Mean launch duration (us) of a 16-byte non-temporal streaming read of
    nbytes, rotating over the device buffers (tensors or raw addresses)."""
    ptrs = (C.c_void_p * len(bufs))(*[b.data_ptr() if isinstance(b, torch.Tensor) else int(b) for b in bufs])
    us = C.c_float(0.0)
    check(lib().csa_debug_stream_read(ptrs, len(bufs), int(nbytes), int(reps), _stream(stream), C.byref(us)))
    return float(us.value)
