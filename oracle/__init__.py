"""Python face of the plain CPU oracle for the MSA decode path.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's CPU-baseline leg
may import this package. It shares no code with the HIP library and never imports it.

The arithmetic lives in msa_oracle.c (fp64, single-threaded); this module only marshals
numpy arrays through ctypes and loops over sequences, tokens and groups. Layouts are the
oracle's logical ones (see msa_oracle.c): index keys codes [T][64] / scales [T][8], K and V
codes [T][4][64] / scales [T][4][8], bf16 values as uint16 bit patterns.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build

_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")

TOPK = 16
BLOCK = 128
D = 128


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    src = os.path.join(os.path.dirname(path), "msa_oracle.c")
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
        _build.build()
    L = ctypes.CDLL(path)
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_value.restype = ctypes.c_double
    L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e2m1_encode_magnitude.restype = ctypes.c_uint8
    L.orc_e2m1_encode_magnitude.argtypes = [ctypes.c_float]
    L.orc_nvfp4_quantize.restype = None
    L.orc_nvfp4_quantize.argtypes = [_f32p, ctypes.c_int64, _u8p, _u8p]
    L.orc_nvfp4_dequantize.restype = None
    L.orc_nvfp4_dequantize.argtypes = [_u8p, _u8p, ctypes.c_int64, _f64p]
    L.orc_bf16_value.restype = ctypes.c_double
    L.orc_bf16_value.argtypes = [ctypes.c_uint16]
    L.orc_index_scores.restype = None
    L.orc_index_scores.argtypes = [_u16p, _u8p, _u8p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, _f64p]
    L.orc_index_scores_lse.restype = None
    L.orc_index_scores_lse.argtypes = L.orc_index_scores.argtypes
    L.orc_block_topk.restype = ctypes.c_int
    L.orc_block_topk.argtypes = [_f64p, ctypes.c_int32, ctypes.c_int32, _i32p,
                                 ctypes.POINTER(ctypes.c_double)]
    L.orc_sparse_attention_token.restype = None
    L.orc_sparse_attention_token.argtypes = [_u16p, _u8p, _u8p, _u8p, _u8p, ctypes.c_int32,
                                             _i32p, ctypes.c_int32, ctypes.c_int64,
                                             ctypes.c_double, _f64p]
    _lib = L
    return L


# ------------------------------------------------------------------ codec

def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(int(b))


def e2m1_value(n: int) -> float:
    return lib().orc_e2m1_value(int(n))


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e2m1_encode_magnitude(r: float) -> int:
    return int(lib().orc_e2m1_encode_magnitude(float(r)))


def quantize(x: np.ndarray):
    """fp32 [..., 128] -> (codes uint8 [..., 64], scales uint8 [..., 8])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    assert x.shape[-1] == D
    n = int(np.prod(lead)) if lead else 1
    codes = np.empty((n, 64), np.uint8)
    scales = np.empty((n, 8), np.uint8)
    lib().orc_nvfp4_quantize(x.reshape(n, D), n, codes, scales)
    return codes.reshape(*lead, 64), scales.reshape(*lead, 8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(codes [..., 64], scales [..., 8]) -> exact fp64 values [..., 128]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    lead = codes.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    out = np.empty((n, D), np.float64)
    lib().orc_nvfp4_dequantize(codes.reshape(n, 64), scales.reshape(n, 8), n, out)
    return out.reshape(*lead, D)


# ------------------------------------------------------------------ indexer and selection

def index_scores(q_idx_bits: np.ndarray, ik_codes: np.ndarray, ik_scales: np.ndarray,
                 T: int, q: int, nb_out: int) -> np.ndarray:
    """Block scores of one sequence: [q][4][nb_out] fp64, -inf where a block has no valid key."""
    q_idx_bits = np.ascontiguousarray(q_idx_bits, dtype=np.uint16).reshape(q, 4, D)
    ik_codes = np.ascontiguousarray(ik_codes[:T], dtype=np.uint8)
    ik_scales = np.ascontiguousarray(ik_scales[:T], dtype=np.uint8)
    out = np.empty((q, 4, nb_out), np.float64)
    lib().orc_index_scores(q_idx_bits, ik_codes, ik_scales, int(T), int(q), int(nb_out), out)
    return out


def index_scores_lse(q_idx_bits: np.ndarray, ik_codes: np.ndarray, ik_scales: np.ndarray,
                     T: int, q: int, nb_out: int) -> np.ndarray:
    """As index_scores, with the block's log-sum-exp of its token scores instead of the max."""
    q_idx_bits = np.ascontiguousarray(q_idx_bits, dtype=np.uint16).reshape(q, 4, D)
    ik_codes = np.ascontiguousarray(ik_codes[:T], dtype=np.uint8)
    ik_scales = np.ascontiguousarray(ik_scales[:T], dtype=np.uint8)
    out = np.empty((q, 4, nb_out), np.float64)
    lib().orc_index_scores_lse(q_idx_bits, ik_codes, ik_scales, int(T), int(q), int(nb_out), out)
    return out


def block_topk(scores_row: np.ndarray, n_eligible: int, topk: int = TOPK):
    """Selected block ids (ascending, -1 padded) and the selection margin of one row."""
    s = np.ascontiguousarray(scores_row[:n_eligible], dtype=np.float64)
    ids = np.empty(topk, np.int32)
    m = ctypes.c_double()
    lib().orc_block_topk(s, int(n_eligible), int(topk), ids, ctypes.byref(m))
    return ids, m.value


def select_sequence(scores: np.ndarray, T: int, q: int, topk: int = TOPK):
    """Per-row selection for one sequence: ids [q][4][topk], margins [q][4]."""
    ids = np.empty((q, 4, topk), np.int32)
    margins = np.empty((q, 4), np.float64)
    for j in range(q):
        p = T - q + j
        n_elig = p // BLOCK + 1
        for g in range(4):
            ids[j, g], margins[j, g] = block_topk(scores[j, g], n_elig, topk)
    return ids, margins


def block_topk_variant(scores_row: np.ndarray, n_eligible: int, topk: int, init_blocks: int,
                       local_blocks: int) -> np.ndarray:
    """Selection with the window knobs of "MiniMax M3 on vLLM", section "MSA mechanism" (the
    config exposes init blocks and local blocks; the current recipe uses 0 and 1): of the
    eligible blocks 0..n-1, the first `init_blocks` and the last `local_blocks` are always kept,
    and the rest of the `topk` places go to the best other blocks by (score descending, index
    ascending); a forced block is never counted twice. With at most `topk` eligible blocks all
    are kept. Ids ascending, padded with -1 to `topk`."""
    n = int(n_eligible)
    if n <= topk:
        kept = list(range(max(n, 0)))
    else:
        forced = set(range(min(init_blocks, n))) | set(range(max(n - local_blocks, 0), n))
        rest = [i for i in range(n) if i not in forced]
        best = sorted(rest, key=lambda i: (-float(scores_row[i]), i))[:topk - len(forced)]
        kept = sorted(forced | set(best))
    return np.array(kept + [-1] * (topk - len(kept)), np.int32)


def dcp_local_topk(scores_row: np.ndarray, n_eligible: int, shard_blocks, topk: int = TOPK):
    """One shard's local candidates of a row ("vLLM day-0 support for MiniMax-M3.1-Flash",
    section "Indexer NVFP4 DCP": each device ranks only its own share of the pages and keeps
    its local top 16 per index head).

    shard_blocks: the block ids the shard holds. Its eligible blocks (id < n_eligible) are
    ranked by (score descending, id ascending), the forced block n_eligible - 1 first when the
    shard holds it; the best `topk` are returned as (ids ascending, forced flags).
    """
    forced = n_eligible - 1
    mine = [int(i) for i in shard_blocks if 0 <= int(i) < n_eligible]
    order = sorted(mine, key=lambda i: (i != forced, -float(scores_row[i]), i))
    kept = sorted(order[:topk])
    return kept, [i == forced for i in kept]


def dcp_merge(scores_row: np.ndarray, n_eligible: int, local_lists, topk: int = TOPK):
    """The owner's merge of the shards' local candidates ("vLLM day-0 support for
    MiniMax-M3.1-Flash", section "Indexer NVFP4 DCP": the local top-16 lists are merged into
    the final top 16): the best `topk` of their union by the same order (forced block first,
    then score descending, id ascending); ids ascending, padded with -1."""
    forced = n_eligible - 1
    union = [i for ids in local_lists for i in ids]
    kept = sorted(sorted(union, key=lambda i: (i != forced, -float(scores_row[i]), i))[:topk])
    return np.array(kept + [-1] * (topk - len(kept)), np.int32)


# ------------------------------------------------------------------ attention

def sparse_attention_token(q_bits, k_codes, k_scales, v_codes, v_scales, T, ids, p, scale):
    """One query token, 64 heads: exact attention over the given block ids per group."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16).reshape(64, D)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(4, -1)
    out = np.empty((64, D), np.float64)
    lib().orc_sparse_attention_token(
        q_bits, np.ascontiguousarray(k_codes, dtype=np.uint8),
        np.ascontiguousarray(k_scales, dtype=np.uint8),
        np.ascontiguousarray(v_codes, dtype=np.uint8),
        np.ascontiguousarray(v_scales, dtype=np.uint8),
        int(T), ids, int(ids.shape[1]), int(p), float(scale), out)
    return out


def dense_ids(p: int) -> np.ndarray:
    """All eligible blocks of a token at position p, for each group: the dense reference."""
    n = p // BLOCK + 1
    return np.tile(np.arange(n, dtype=np.int32), (4, 1))


def default_scale() -> float:
    return 1.0 / math.sqrt(D)
