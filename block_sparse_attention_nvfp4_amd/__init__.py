"""MiniMax Sparse Attention (MSA) decode path with NVFP4 caches for AMD MI355X (gfx950).

Thin Python binding of libmsa.so (C ABI in include/msa.h). Every step of the path runs in the
library's HIP kernels; this module only marshals torch tensors (device memory) and the current
HIP stream into the C calls, with the same names:

    msa_kv_insert_nvfp4(cache, slots, k, v, ik)
    msa_indexer_score(cache, batch, q_idx, block_scores)
    msa_indexer_score_ex(cache, batch, q_idx, reduction, block_scores)   # max or log-sum-exp
    msa_indexer_score_shared_prefix(cache, batch, q_idx, prefix_blocks, block_scores)
    msa_block_topk(block_scores, batch, topk, block_ids)
    msa_block_topk_window(block_scores, batch, topk, init_blocks, local_blocks, block_ids)
    msa_block_topk_local(shard_scores, block_begin, block_stride, batch, topk, cand_ids,
                         cand_keys)           # one shard's local lists (context parallelism)
    msa_block_topk_merge(cand_ids, cand_keys, batch, topk, block_ids)   # merge of all shards
    msa_sparse_attn_workspace_bytes(batch)
    msa_sparse_attn_decode(cache, batch, q, block_ids, softmax_scale, out, workspace)
    msa_sparse_attn_decode_topk(cache, batch, q, block_ids, softmax_scale, out, workspace)
                                             # rows of 1..64 ids (block_ids' last dimension)
    msa_select_attn_decode(cache, batch, block_scores, topk, block_ids, q, softmax_scale, out,
                           workspace)        # the last two in one launch
    msa_insert_indexer_score(cache, batch, k, v, ik, q_idx, block_scores)  # insert + indexer
    msa_decode_step(cache, batch, k, v, ik, q_idx, q, topk, softmax_scale, block_scores,
                    block_ids, out, workspace)   # the two launches above and below in one call
    msa_decode_step_noalloc(cache, batch, k, v, ik, q_idx, q, topk, softmax_scale, block_scores,
                            block_ids, out)     # the same with the library's static workspace
    use_library(checked), msa_debug_checks()   # the checked build and its failed-check counts

A non-zero status raises MSAError. There is no fallback: importing fails loudly when the
library has not been built (python block_sparse_attention_nvfp4_amd/build.py).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa.so")
# the same library built with the kernels' checks (include/msa_debug.h): use_library(True)
CHECKED_LIB_PATH = os.path.join(HERE, "libmsa_checked.so")

BLOCK = 128
HEAD_DIM = 128
KV_HEADS = 4
Q_HEADS = 64
TOPK = 16
HEAD_PAGE_BYTES = 9216

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_WORKSPACE = -3
MSA_ERR_HIP = -4
MSA_REDUCE_MAX = 0
MSA_REDUCE_LSE = 1

EXPORTED = ("msa_page_bytes", "msa_kv_insert_nvfp4", "msa_indexer_score", "msa_indexer_score_ex",
            "msa_indexer_score_shared_prefix", "msa_indexer_score_shard",
            "msa_block_topk",
            "msa_block_topk_window", "msa_block_topk_local", "msa_block_topk_merge",
            "msa_sparse_attn_workspace_bytes", "msa_sparse_attn_decode",
            "msa_sparse_attn_decode_topk", "msa_select_attn_decode",
            "msa_sparse_attn_shared_prefix_workspace_bytes", "msa_sparse_attn_decode_shared_prefix",
            "msa_insert_indexer_score", "msa_decode_step", "msa_decode_step_window",
            "msa_decode_step_noalloc",
            "msa_last_error", "msa_version",
            # include/msa_debug.h (checked build diagnostics)
            "msa_debug_checks",
            # include/msa_probe.h (measurement aid)
            "msa_probe_stream_read", "msa_probe_sink_words")


class MSAError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("ik", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64)]


class _Batch(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("ctx_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("q_len", ctypes.c_int32)]


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python block_sparse_attention_nvfp4_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.msa_page_bytes.restype, L.msa_page_bytes.argtypes = sz, [ctypes.c_int]
    L.msa_kv_insert_nvfp4.restype = ctypes.c_int
    L.msa_kv_insert_nvfp4.argtypes = [ctypes.POINTER(_Cache), vp, vp, vp, vp, i32, vp]
    L.msa_indexer_score.restype = ctypes.c_int
    L.msa_indexer_score.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, vp, vp]
    L.msa_indexer_score_ex.restype = ctypes.c_int
    L.msa_indexer_score_ex.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, i32, vp,
                                       vp]
    L.msa_indexer_score_shared_prefix.restype = ctypes.c_int
    L.msa_indexer_score_shared_prefix.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch),
                                                  vp, i32, vp, vp]
    L.msa_indexer_score_shard.restype = ctypes.c_int
    L.msa_indexer_score_shard.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), i32, i32,
                                          i32, vp, vp, vp]
    L.msa_block_topk.restype = ctypes.c_int
    L.msa_block_topk.argtypes = [vp, ctypes.POINTER(_Batch), i32, vp, vp]
    L.msa_block_topk_window.restype = ctypes.c_int
    L.msa_block_topk_window.argtypes = [vp, ctypes.POINTER(_Batch), i32, i32, i32, vp, vp]
    L.msa_block_topk_local.restype = ctypes.c_int
    L.msa_block_topk_local.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(_Batch), i32, vp, vp,
                                       vp]
    L.msa_block_topk_merge.restype = ctypes.c_int
    L.msa_block_topk_merge.argtypes = [vp, vp, i32, ctypes.POINTER(_Batch), i32, vp, vp]
    L.msa_sparse_attn_workspace_bytes.restype = sz
    L.msa_sparse_attn_workspace_bytes.argtypes = [ctypes.POINTER(_Batch)]
    L.msa_sparse_attn_decode.restype = ctypes.c_int
    L.msa_sparse_attn_decode.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, vp,
                                         ctypes.c_float, vp, vp, sz, vp]
    L.msa_sparse_attn_decode_topk.restype = ctypes.c_int
    L.msa_sparse_attn_decode_topk.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp,
                                              vp, i32, ctypes.c_float, vp, vp, sz, vp]
    L.msa_sparse_attn_shared_prefix_workspace_bytes.restype = sz
    L.msa_sparse_attn_shared_prefix_workspace_bytes.argtypes = [ctypes.POINTER(_Batch)]
    L.msa_sparse_attn_decode_shared_prefix.restype = ctypes.c_int
    L.msa_sparse_attn_decode_shared_prefix.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch),
                                                       vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    L.msa_select_attn_decode.restype = ctypes.c_int
    L.msa_select_attn_decode.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, i32,
                                         vp, vp, ctypes.c_float, vp, vp, sz, vp]
    L.msa_insert_indexer_score.restype = ctypes.c_int
    L.msa_insert_indexer_score.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, vp,
                                           vp, vp, vp, vp]
    L.msa_decode_step.restype = ctypes.c_int
    L.msa_decode_step.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, vp, vp, vp,
                                  vp, i32, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    L.msa_decode_step_window.restype = ctypes.c_int
    L.msa_decode_step_window.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, vp,
                                         vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp, vp,
                                         vp, sz, vp]
    L.msa_decode_step_noalloc.restype = ctypes.c_int
    L.msa_decode_step_noalloc.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), vp, vp,
                                          vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp]
    L.msa_probe_stream_read.restype = ctypes.c_int
    L.msa_probe_stream_read.argtypes = [vp, sz, vp, vp]
    L.msa_probe_sink_words.restype, L.msa_probe_sink_words.argtypes = sz, []
    L.msa_last_error.restype, L.msa_last_error.argtypes = ctypes.c_char_p, []
    L.msa_version.restype, L.msa_version.argtypes = ctypes.c_char_p, []
    L.msa_debug_checks.restype = ctypes.c_int
    L.msa_debug_checks.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    return L


lib = _load()
_libs = {False: lib}


def use_library(checked: bool) -> None:
    """Route every call of this module to libmsa_checked.so (True) or libmsa.so (False). Both
    are built from the same sources; the checked one also counts failed kernel checks, which
    msa_debug_checks() returns."""
    global lib
    if checked not in _libs:
        _libs[checked] = _load(CHECKED_LIB_PATH)
    lib = _libs[checked]


def msa_debug_checks():
    """(failed checks, lowest failing site) on the current device since the previous call, both
    reset; only the checked library counts (MSAError from libmsa.so)."""
    count, site = ctypes.c_uint32(0), ctypes.c_uint32(0)
    _check(lib.msa_debug_checks(ctypes.byref(count), ctypes.byref(site)))
    return int(count.value), int(site.value)


def _check(rc: int) -> None:
    if rc != MSA_OK:
        raise MSAError(rc, lib.msa_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype: torch.dtype, name: str):
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Cache:
    """Paged NVFP4 pools (K, V, index keys) as device uint8 tensors; see include/msa.h."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, ik: torch.Tensor):
        self.k, self.v, self.ik = k, v, ik
        self.num_pages = int(ik.shape[0])
        self._c = _Cache(_ptr(k, torch.uint8, "k"), _ptr(v, torch.uint8, "v"),
                         _ptr(ik, torch.uint8, "ik"), self.num_pages)

    @classmethod
    def allocate(cls, num_pages: int, device="cuda") -> "Cache":
        """Zero-initialized pools for `num_pages` pages."""
        shape = (num_pages, KV_HEADS, HEAD_PAGE_BYTES)
        return cls(torch.zeros(shape, dtype=torch.uint8, device=device),
                   torch.zeros(shape, dtype=torch.uint8, device=device),
                   torch.zeros((num_pages, HEAD_PAGE_BYTES), dtype=torch.uint8, device=device))


class Batch:
    """Block table (int32 [batch][max_blocks]), context lengths (int32 [batch]) and q_len."""

    def __init__(self, block_table: torch.Tensor, ctx_lens: torch.Tensor, q_len: int):
        if block_table.dim() != 2 or ctx_lens.dim() != 1 or ctx_lens.shape[0] != block_table.shape[0]:
            raise ValueError("block_table must be [batch][max_blocks] and ctx_lens [batch]")
        self.block_table, self.ctx_lens, self.q_len = block_table, ctx_lens, int(q_len)
        self.batch, self.max_blocks = int(block_table.shape[0]), int(block_table.shape[1])
        self._c = _Batch(_ptr(block_table, torch.int32, "block_table"),
                         _ptr(ctx_lens, torch.int32, "ctx_lens"), self.batch, self.max_blocks,
                         self.q_len)

    @property
    def rows(self) -> int:
        return self.batch * self.q_len


def msa_page_bytes(which: int) -> int:
    return int(lib.msa_page_bytes(int(which)))


def msa_version() -> str:
    return lib.msa_version().decode()


def msa_last_error() -> str:
    return lib.msa_last_error().decode()


def msa_kv_insert_nvfp4(cache: Cache, slots: torch.Tensor, k: Optional[torch.Tensor],
                        v: Optional[torch.Tensor], ik: Optional[torch.Tensor], stream=None) -> None:
    n = int(slots.shape[0])
    for name, t, tail in (("k", k, (KV_HEADS, HEAD_DIM)), ("v", v, (KV_HEADS, HEAD_DIM)),
                          ("ik", ik, (HEAD_DIM,))):
        if t is not None and tuple(t.shape) != (n, *tail):
            raise ValueError(f"{name}: expected shape {(n, *tail)}, got {tuple(t.shape)}")
    _check(lib.msa_kv_insert_nvfp4(ctypes.byref(cache._c), _ptr(slots, torch.int64, "slots"),
                                   _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
                                   _ptr(ik, torch.float32, "ik"), n, _stream(stream)))


def msa_indexer_score(cache: Cache, batch: Batch, q_idx: torch.Tensor, block_scores: torch.Tensor,
                      stream=None) -> None:
    if tuple(q_idx.shape) != (batch.rows, KV_HEADS, HEAD_DIM):
        raise ValueError(f"q_idx: expected {(batch.rows, KV_HEADS, HEAD_DIM)}, got {tuple(q_idx.shape)}")
    if tuple(block_scores.shape) != (batch.rows, KV_HEADS, batch.max_blocks):
        raise ValueError("block_scores: expected [batch*q_len][4][max_blocks]")
    _check(lib.msa_indexer_score(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                 _ptr(q_idx, torch.bfloat16, "q_idx"),
                                 _ptr(block_scores, torch.float32, "block_scores"), _stream(stream)))


def msa_indexer_score_ex(cache: Cache, batch: Batch, q_idx: torch.Tensor, reduction: int,
                         block_scores: torch.Tensor, stream=None) -> None:
    if tuple(q_idx.shape) != (batch.rows, KV_HEADS, HEAD_DIM):
        raise ValueError(f"q_idx: expected {(batch.rows, KV_HEADS, HEAD_DIM)}, got {tuple(q_idx.shape)}")
    if tuple(block_scores.shape) != (batch.rows, KV_HEADS, batch.max_blocks):
        raise ValueError("block_scores: expected [batch*q_len][4][max_blocks]")
    _check(lib.msa_indexer_score_ex(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                    _ptr(q_idx, torch.bfloat16, "q_idx"), int(reduction),
                                    _ptr(block_scores, torch.float32, "block_scores"),
                                    _stream(stream)))


def msa_indexer_score_shared_prefix(cache: Cache, batch: Batch, q_idx: torch.Tensor,
                                    prefix_blocks: int, block_scores: torch.Tensor,
                                    stream=None) -> None:
    if tuple(q_idx.shape) != (batch.rows, KV_HEADS, HEAD_DIM):
        raise ValueError(f"q_idx: expected {(batch.rows, KV_HEADS, HEAD_DIM)}, got {tuple(q_idx.shape)}")
    if tuple(block_scores.shape) != (batch.rows, KV_HEADS, batch.max_blocks):
        raise ValueError("block_scores: expected [batch*q_len][4][max_blocks]")
    _check(lib.msa_indexer_score_shared_prefix(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                               _ptr(q_idx, torch.bfloat16, "q_idx"),
                                               int(prefix_blocks),
                                               _ptr(block_scores, torch.float32, "block_scores"),
                                               _stream(stream)))


def msa_indexer_score_shard(cache: Cache, shard: Batch, block_begin: int, block_stride: int,
                            total_blocks: int, q_idx: torch.Tensor, shard_scores: torch.Tensor,
                            stream=None) -> None:
    """shard: a Batch whose table column c holds the page of global block
    block_begin + c * block_stride; shard_scores: [batch*q_len][4][shard.max_blocks]."""
    if tuple(q_idx.shape) != (shard.rows, KV_HEADS, HEAD_DIM):
        raise ValueError(f"q_idx: expected {(shard.rows, KV_HEADS, HEAD_DIM)}, got {tuple(q_idx.shape)}")
    if tuple(shard_scores.shape) != (shard.rows, KV_HEADS, shard.max_blocks):
        raise ValueError("shard_scores: expected [batch*q_len][4][max_blocks of the shard]")
    _check(lib.msa_indexer_score_shard(ctypes.byref(cache._c), ctypes.byref(shard._c),
                                       int(block_begin), int(block_stride), int(total_blocks),
                                       _ptr(q_idx, torch.bfloat16, "q_idx"),
                                       _ptr(shard_scores, torch.float32, "shard_scores"),
                                       _stream(stream)))


def msa_block_topk(block_scores: torch.Tensor, batch: Batch, topk: int, block_ids: torch.Tensor,
                   stream=None) -> None:
    if tuple(block_scores.shape) != (batch.rows, KV_HEADS, batch.max_blocks):
        raise ValueError("block_scores: expected [batch*q_len][4][max_blocks]")
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, int(topk)):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    _check(lib.msa_block_topk(_ptr(block_scores, torch.float32, "block_scores"),
                              ctypes.byref(batch._c), int(topk),
                              _ptr(block_ids, torch.int32, "block_ids"), _stream(stream)))


def msa_block_topk_window(block_scores: torch.Tensor, batch: Batch, topk: int, init_blocks: int,
                          local_blocks: int, block_ids: torch.Tensor, stream=None) -> None:
    if tuple(block_scores.shape) != (batch.rows, KV_HEADS, batch.max_blocks):
        raise ValueError("block_scores: expected [batch*q_len][4][max_blocks]")
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, int(topk)):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    _check(lib.msa_block_topk_window(_ptr(block_scores, torch.float32, "block_scores"),
                                     ctypes.byref(batch._c), int(topk), int(init_blocks),
                                     int(local_blocks), _ptr(block_ids, torch.int32, "block_ids"),
                                     _stream(stream)))


def msa_block_topk_local(shard_scores: torch.Tensor, block_begin: int, block_stride: int,
                         batch: Batch, topk: int, cand_ids: torch.Tensor, cand_keys: torch.Tensor,
                         stream=None) -> None:
    """shard_scores: [batch*q_len][4][n_cols] fp32 whose columns are contiguous; its row stride
    may be larger (a column slice of msa_indexer_score's output passes as it is)."""
    if shard_scores.dim() != 3 or tuple(shard_scores.shape[:2]) != (batch.rows, KV_HEADS):
        raise ValueError("shard_scores: expected [batch*q_len][4][n_cols]")
    n_cols = int(shard_scores.shape[2])
    ld = int(shard_scores.stride(1))
    if shard_scores.dtype != torch.float32 or not shard_scores.is_cuda:
        raise TypeError("shard_scores: expected a float32 device tensor")
    if shard_scores.stride(2) != 1 or shard_scores.stride(0) != KV_HEADS * ld or ld < n_cols:
        raise ValueError("shard_scores: columns must be contiguous, rows evenly spaced")
    for name, t in (("cand_ids", cand_ids), ("cand_keys", cand_keys)):
        if tuple(t.shape) != (batch.rows, KV_HEADS, int(topk)):
            raise ValueError(f"{name}: expected [batch*q_len][4][topk]")
    _check(lib.msa_block_topk_local(shard_scores.data_ptr(), ld, int(block_begin),
                                    int(block_stride), n_cols, ctypes.byref(batch._c), int(topk),
                                    _ptr(cand_ids, torch.int32, "cand_ids"),
                                    _ptr(cand_keys, torch.int32, "cand_keys"), _stream(stream)))


def msa_block_topk_merge(cand_ids: torch.Tensor, cand_keys: torch.Tensor, batch: Batch, topk: int,
                         block_ids: torch.Tensor, stream=None) -> None:
    """cand_ids, cand_keys: [n_shards][batch*q_len][4][topk] (rank keys as int32 bit patterns)."""
    n_shards = int(cand_ids.shape[0]) if cand_ids.dim() == 4 else -1
    for name, t in (("cand_ids", cand_ids), ("cand_keys", cand_keys)):
        if tuple(t.shape) != (n_shards, batch.rows, KV_HEADS, int(topk)):
            raise ValueError(f"{name}: expected [n_shards][batch*q_len][4][topk]")
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, int(topk)):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    _check(lib.msa_block_topk_merge(_ptr(cand_ids, torch.int32, "cand_ids"),
                                    _ptr(cand_keys, torch.int32, "cand_keys"), n_shards,
                                    ctypes.byref(batch._c), int(topk),
                                    _ptr(block_ids, torch.int32, "block_ids"), _stream(stream)))


def msa_sparse_attn_workspace_bytes(batch: Batch) -> int:
    return int(lib.msa_sparse_attn_workspace_bytes(ctypes.byref(batch._c)))


def msa_sparse_attn_decode(cache: Cache, batch: Batch, q: torch.Tensor, block_ids: torch.Tensor,
                           softmax_scale: float, out: torch.Tensor,
                           workspace: Optional[torch.Tensor], stream=None) -> None:
    if tuple(q.shape) != (batch.rows, Q_HEADS, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out: expected [batch*q_len][64][128]")
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, TOPK):
        raise ValueError("block_ids: expected [batch*q_len][4][16]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.msa_sparse_attn_decode(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                      _ptr(q, torch.bfloat16, "q"),
                                      _ptr(block_ids, torch.int32, "block_ids"),
                                      float(softmax_scale), _ptr(out, torch.bfloat16, "out"),
                                      ws_ptr, ws_bytes, _stream(stream)))


def msa_sparse_attn_decode_topk(cache: Cache, batch: Batch, q: torch.Tensor,
                                block_ids: torch.Tensor, softmax_scale: float, out: torch.Tensor,
                                workspace: Optional[torch.Tensor], stream=None) -> None:
    """Attention over rows of any selection size: block_ids is [batch*q_len][4][topk], and topk
    is taken from its last dimension."""
    if tuple(q.shape) != (batch.rows, Q_HEADS, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out: expected [batch*q_len][64][128]")
    if block_ids.dim() != 3 or tuple(block_ids.shape[:2]) != (batch.rows, KV_HEADS):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.msa_sparse_attn_decode_topk(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                           _ptr(q, torch.bfloat16, "q"),
                                           _ptr(block_ids, torch.int32, "block_ids"),
                                           int(block_ids.shape[2]), float(softmax_scale),
                                           _ptr(out, torch.bfloat16, "out"), ws_ptr, ws_bytes,
                                           _stream(stream)))


def msa_sparse_attn_shared_prefix_workspace_bytes(batch: Batch) -> int:
    return int(lib.msa_sparse_attn_shared_prefix_workspace_bytes(ctypes.byref(batch._c)))


def msa_sparse_attn_decode_shared_prefix(cache: Cache, batch: Batch, q: torch.Tensor,
                                         block_ids: torch.Tensor, prefix_blocks: int,
                                         softmax_scale: float, out: torch.Tensor,
                                         workspace: torch.Tensor, stream=None) -> None:
    if tuple(q.shape) != (batch.rows, Q_HEADS, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out: expected [batch*q_len][64][128]")
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, TOPK):
        raise ValueError("block_ids: expected [batch*q_len][4][16]")
    _check(lib.msa_sparse_attn_decode_shared_prefix(
        ctypes.byref(cache._c), ctypes.byref(batch._c), _ptr(q, torch.bfloat16, "q"),
        _ptr(block_ids, torch.int32, "block_ids"), int(prefix_blocks), float(softmax_scale),
        _ptr(out, torch.bfloat16, "out"), _ptr(workspace, workspace.dtype, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def msa_select_attn_decode(cache: Cache, batch: Batch, block_scores: torch.Tensor, topk: int,
                           block_ids: torch.Tensor, q: torch.Tensor, softmax_scale: float,
                           out: torch.Tensor, workspace: Optional[torch.Tensor],
                           stream=None) -> None:
    if tuple(block_scores.shape) != (batch.rows, KV_HEADS, batch.max_blocks):
        raise ValueError("block_scores: expected [batch*q_len][4][max_blocks]")
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, int(topk)):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    if tuple(q.shape) != (batch.rows, Q_HEADS, HEAD_DIM) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out: expected [batch*q_len][64][128]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.msa_select_attn_decode(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                      _ptr(block_scores, torch.float32, "block_scores"), int(topk),
                                      _ptr(block_ids, torch.int32, "block_ids"),
                                      _ptr(q, torch.bfloat16, "q"), float(softmax_scale),
                                      _ptr(out, torch.bfloat16, "out"), ws_ptr, ws_bytes,
                                      _stream(stream)))


def _check_step_shapes(batch: Batch, **tensors) -> None:
    n = batch.rows
    tails = dict(k=(KV_HEADS, HEAD_DIM), v=(KV_HEADS, HEAD_DIM), ik=(HEAD_DIM,),
                 q_idx=(KV_HEADS, HEAD_DIM), q=(Q_HEADS, HEAD_DIM), out=(Q_HEADS, HEAD_DIM),
                 block_scores=(KV_HEADS, batch.max_blocks), block_ids=(KV_HEADS, TOPK))
    for name, t in tensors.items():
        if tuple(t.shape) != (n, *tails[name]):
            raise ValueError(f"{name}: expected shape {(n, *tails[name])}, got {tuple(t.shape)}")


def msa_insert_indexer_score(cache: Cache, batch: Batch, k: torch.Tensor, v: torch.Tensor,
                             ik: torch.Tensor, q_idx: torch.Tensor, block_scores: torch.Tensor,
                             stream=None) -> None:
    _check_step_shapes(batch, k=k, v=v, ik=ik, q_idx=q_idx, block_scores=block_scores)
    _check(lib.msa_insert_indexer_score(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                        _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
                                        _ptr(ik, torch.float32, "ik"),
                                        _ptr(q_idx, torch.bfloat16, "q_idx"),
                                        _ptr(block_scores, torch.float32, "block_scores"),
                                        _stream(stream)))


def msa_decode_step(cache: Cache, batch: Batch, k: torch.Tensor, v: torch.Tensor,
                    ik: torch.Tensor, q_idx: torch.Tensor, q: torch.Tensor, topk: int,
                    softmax_scale: float, block_scores: torch.Tensor, block_ids: torch.Tensor,
                    out: torch.Tensor, workspace: Optional[torch.Tensor], stream=None) -> None:
    _check_step_shapes(batch, k=k, v=v, ik=ik, q_idx=q_idx, q=q, out=out,
                       block_scores=block_scores)
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, int(topk)):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.msa_decode_step(ctypes.byref(cache._c), ctypes.byref(batch._c),
                               _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
                               _ptr(ik, torch.float32, "ik"), _ptr(q_idx, torch.bfloat16, "q_idx"),
                               _ptr(q, torch.bfloat16, "q"), int(topk), float(softmax_scale),
                               _ptr(block_scores, torch.float32, "block_scores"),
                               _ptr(block_ids, torch.int32, "block_ids"),
                               _ptr(out, torch.bfloat16, "out"), ws_ptr, ws_bytes,
                               _stream(stream)))


def msa_decode_step_window(cache: Cache, batch: Batch, k: torch.Tensor, v: torch.Tensor,
                           ik: torch.Tensor, q_idx: torch.Tensor, q: torch.Tensor, topk: int,
                           init_blocks: int, local_blocks: int, softmax_scale: float,
                           block_scores: torch.Tensor, block_ids: torch.Tensor, out: torch.Tensor,
                           workspace: Optional[torch.Tensor], stream=None) -> None:
    """The decode step with the window knobs: insert + indexer, msa_block_topk_window, then
    attention over the topk ids per row."""
    _check_step_shapes(batch, k=k, v=v, ik=ik, q_idx=q_idx, q=q, out=out,
                       block_scores=block_scores)
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, int(topk)):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.msa_decode_step_window(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                      _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
                                      _ptr(ik, torch.float32, "ik"),
                                      _ptr(q_idx, torch.bfloat16, "q_idx"),
                                      _ptr(q, torch.bfloat16, "q"), int(topk), int(init_blocks),
                                      int(local_blocks), float(softmax_scale),
                                      _ptr(block_scores, torch.float32, "block_scores"),
                                      _ptr(block_ids, torch.int32, "block_ids"),
                                      _ptr(out, torch.bfloat16, "out"), ws_ptr, ws_bytes,
                                      _stream(stream)))


def msa_decode_step_noalloc(cache: Cache, batch: Batch, k: torch.Tensor, v: torch.Tensor,
                            ik: torch.Tensor, q_idx: torch.Tensor, q: torch.Tensor, topk: int,
                            softmax_scale: float, block_scores: torch.Tensor,
                            block_ids: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """msa_decode_step with the library's static workspace (no workspace argument)."""
    _check_step_shapes(batch, k=k, v=v, ik=ik, q_idx=q_idx, q=q, out=out,
                       block_scores=block_scores)
    if tuple(block_ids.shape) != (batch.rows, KV_HEADS, int(topk)):
        raise ValueError("block_ids: expected [batch*q_len][4][topk]")
    _check(lib.msa_decode_step_noalloc(ctypes.byref(cache._c), ctypes.byref(batch._c),
                                       _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"),
                                       _ptr(ik, torch.float32, "ik"),
                                       _ptr(q_idx, torch.bfloat16, "q_idx"),
                                       _ptr(q, torch.bfloat16, "q"), int(topk),
                                       float(softmax_scale),
                                       _ptr(block_scores, torch.float32, "block_scores"),
                                       _ptr(block_ids, torch.int32, "block_ids"),
                                       _ptr(out, torch.bfloat16, "out"), _stream(stream)))


def msa_probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement aid (include/msa_probe.h): read every byte of `buf` once from HBM."""
    if not buf.is_cuda or not buf.is_contiguous() or sink.dtype != torch.int32 or \
            sink.numel() < msa_probe_sink_words():
        raise ValueError("buf: contiguous device tensor; sink: int32 of msa_probe_sink_words()")
    rc = lib.msa_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                   _ptr(sink, torch.int32, "sink"), _stream(stream))
    if rc != MSA_OK:
        raise MSAError(rc, "msa_probe_stream_read: NULL pointer, misaligned buffer or launch error")


def msa_probe_sink_words() -> int:
    return int(lib.msa_probe_sink_words())


def default_softmax_scale() -> float:
    return 1.0 / math.sqrt(HEAD_DIM)


class DecodeStep:
    """Buffers and the calls of one MSA decode step for a fixed batch shape. mode "step": one
    msa_decode_step call (two launches); "select": insert, indexer, then selection and attention
    in one launch; "separate": the four calls. All three give the same bytes."""

    MODES = ("step", "select", "separate")

    def __init__(self, cache: Cache, batch: Batch, device="cuda", mode: str = "step"):
        if mode not in self.MODES:
            raise ValueError(f"mode must be one of {self.MODES}")
        self.cache, self.batch, self.mode = cache, batch, mode
        rows = batch.rows
        self.block_scores = torch.empty((rows, KV_HEADS, batch.max_blocks), dtype=torch.float32,
                                        device=device)
        self.block_ids = torch.empty((rows, KV_HEADS, TOPK), dtype=torch.int32, device=device)
        self.out = torch.empty((rows, Q_HEADS, HEAD_DIM), dtype=torch.bfloat16, device=device)
        ws = msa_sparse_attn_workspace_bytes(batch)
        # zero-filled once: the attention leaves its counters at zero after every call
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=device) if ws else None

    def run(self, slots, k, v, ik, q_idx, q, softmax_scale=None, stream=None):
        """slots: the new tokens' cache slots (page * 128 + token), used by the modes that call
        msa_kv_insert_nvfp4; they must be the slots of positions T_b - q_len + j, which
        msa_decode_step derives itself."""
        scale = default_softmax_scale() if softmax_scale is None else softmax_scale
        if self.mode == "step":
            msa_decode_step(self.cache, self.batch, k, v, ik, q_idx, q, TOPK, scale,
                            self.block_scores, self.block_ids, self.out, self.workspace, stream)
            return self.out
        msa_kv_insert_nvfp4(self.cache, slots, k, v, ik, stream)
        msa_indexer_score(self.cache, self.batch, q_idx, self.block_scores, stream)
        if self.mode == "select":
            msa_select_attn_decode(self.cache, self.batch, self.block_scores, TOPK, self.block_ids,
                                   q, scale, self.out, self.workspace, stream)
        else:
            msa_block_topk(self.block_scores, self.batch, TOPK, self.block_ids, stream)
            msa_sparse_attn_decode(self.cache, self.batch, q, self.block_ids, scale, self.out,
                                   self.workspace, stream)
        return self.out
