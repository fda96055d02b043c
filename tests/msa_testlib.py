"""Test helpers: run a workload through the HIP path and through the oracle, and compare.

The page-layout readers below restate the byte order documented in include/msa.h in numpy, so
the GPU caches can be compared element by element with the oracle's logical arrays. Nothing here
is shared with the HIP library or the oracle's arithmetic.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import msa_inputs as mi

BLOCK = 128
ATOL = 2e-3     # attention: |gpu - oracle| <= ATOL + RTOL * |oracle| element-wise
RTOL = 1e-2
REL_L2 = 1e-2   # and ||gpu - oracle||_2 / ||oracle||_2 <= REL_L2 per checked set
MARGIN = 1e-3   # rows whose oracle selection margin is at least this must select bit-exactly

# ------------------------------------------------------------------ page layouts (msa.h)
_t = np.arange(128)[:, None]
_e_even = np.arange(0, 128, 2)[None, :]
_g = np.arange(8)[None, :]
ROW_CODE_IDX = ((_t % 32) // 4) * 1024 + 256 * (_e_even // 32) + 64 * (_t // 32) + 16 * (_t % 4) + (_e_even % 32) // 2
ROW_SCALE_IDX = 8192 + (_g // 2) * 256 + (_t // 32) * 64 + (_t % 4) * 16 + ((_t % 32) // 4) * 2 + _g % 2
COL_SCALE_IDX = 8192 + _g * 128 + _t


def unpack_row_page(page: np.ndarray):
    """9,216-byte K / index-key head page -> logical codes [128][64], scales [128][8]."""
    return page[ROW_CODE_IDX], page[ROW_SCALE_IDX]


def unpack_col_page(page: np.ndarray):
    """9,216-byte V head page -> logical codes [128][64], scales [128][8]."""
    e = np.arange(128)
    t = np.arange(128)
    byte = page[e[:, None] * 64 + t[None, :] // 2]                  # [e][t]
    nib = (byte >> (4 * (t[None, :] % 2))) & 15                      # [e][t]
    nib = nib.T.astype(np.uint8)                                     # [t][e]
    codes = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return codes, page[COL_SCALE_IDX]


def gpu_sequence_caches(cache, w: mi.Workload, b: int):
    """Logical (codes, scales) of sequence b read back from the GPU pools: ik [T][64]/[T][8],
    k and v [T][4][64]/[T][4][8]."""
    T = w.ctx_lens[b]
    nb = w.n_blocks(b)
    pages = w.block_table[b, :nb].astype(np.int64)
    ikp = cache.ik[torch.from_numpy(pages).to(cache.ik.device)].cpu().numpy()
    kp = cache.k[torch.from_numpy(pages).to(cache.k.device)].cpu().numpy()
    vp = cache.v[torch.from_numpy(pages).to(cache.v.device)].cpu().numpy()
    out = {}
    c, s = zip(*[unpack_row_page(ikp[i]) for i in range(nb)])
    out["ik"] = (np.concatenate(c)[:T], np.concatenate(s)[:T])
    for name, pool, fn in (("k", kp, unpack_row_page), ("v", vp, unpack_col_page)):
        cs, ss = [], []
        for i in range(nb):
            per_head = [fn(pool[i, h]) for h in range(4)]
            cs.append(np.stack([x[0] for x in per_head], axis=1))
            ss.append(np.stack([x[1] for x in per_head], axis=1))
        out[name] = (np.concatenate(cs)[:T], np.concatenate(ss)[:T])
    return out


# ------------------------------------------------------------------ GPU side
class DeviceWorkload:
    def __init__(self, w: mi.Workload, device: str = "cuda", chunk: int = 1 << 15,
                 mode: str = "step", snapshot: bool = False, fill: int = 0):
        import block_sparse_attention_nvfp4_amd as msa
        self.msa = msa
        self.w = w
        self.cache = msa.Cache.allocate(w.num_pages, device)
        if fill:
            # every byte no insert writes keeps this value (0xFF: E4M3 NaN scales, -6 codes)
            for t in (self.cache.k, self.cache.v, self.cache.ik):
                t.fill_(fill)
        self.table = torch.from_numpy(w.block_table).to(device)
        self.ctx = torch.tensor(w.ctx_lens, dtype=torch.int32, device=device)
        self.batch = msa.Batch(self.table, self.ctx, w.q_len)
        q = w.q_len
        # cached prefix: every token but the q query tokens of each sequence
        for b in range(w.batch):
            T = w.ctx_lens[b]
            for t0 in range(0, T - q, chunk):
                t1 = min(T - q, t0 + chunk)
                self.insert(b, t0, t1)
        # the pools holding the cached prefix only (snapshot=True), to run the step again from
        self.prefix = ([t.clone() for t in (self.cache.k, self.cache.v, self.cache.ik)]
                       if snapshot else None)
        # the step's new tokens, request-major
        toks = [(b, w.ctx_lens[b] - q, w.ctx_lens[b]) for b in range(w.batch)]
        self.new_slots = torch.from_numpy(np.concatenate([w.slots(b, t0, t1) for b, t0, t1 in toks])).to(device)
        self.new_k = torch.cat([w.kv_rows("k", b, t0, t1, device) for b, t0, t1 in toks])
        self.new_v = torch.cat([w.kv_rows("v", b, t0, t1, device) for b, t0, t1 in toks])
        self.new_ik = torch.cat([w.ik_rows(b, t0, t1, device) for b, t0, t1 in toks])
        self.q_idx = w.q_idx.to(device)
        self.q = w.q.to(device)
        self.step = msa.DecodeStep(self.cache, self.batch, device, mode=mode)

    def insert(self, b: int, t0: int, t1: int):
        w, dev = self.w, self.cache.ik.device
        slots = torch.from_numpy(w.slots(b, t0, t1)).to(dev)
        self.msa.msa_kv_insert_nvfp4(self.cache, slots, w.kv_rows("k", b, t0, t1, dev),
                                     w.kv_rows("v", b, t0, t1, dev), w.ik_rows(b, t0, t1, dev))

    def restore_prefix(self):
        for dst, src in zip((self.cache.k, self.cache.v, self.cache.ik), self.prefix):
            dst.copy_(src)

    def run(self):
        out = self.step.run(self.new_slots, self.new_k, self.new_v, self.new_ik, self.q_idx, self.q)
        torch.cuda.synchronize()
        return out


# ------------------------------------------------------------------ oracle side
def oracle_sequence(w: mi.Workload, b: int, attention_tokens: Optional[Sequence[int]] = None,
                    ids_override: Optional[np.ndarray] = None, scale: Optional[float] = None):
    """Oracle reference for sequence b: scores [q][4][max_blocks], ids [q][4][16], margins
    [q][4], and attention [len(tokens)][64][128] for the requested query tokens j."""
    import oracle
    T, q = w.ctx_lens[b], w.q_len
    ik = w.ik_rows(b, 0, T).numpy()
    ikc, iks = oracle.quantize(ik)
    qi = mi.bf16_bits(w.q_idx[b * q:(b + 1) * q])
    scores = oracle.index_scores(qi, ikc, iks, T, q, w.max_blocks)
    ids, margins = oracle.select_sequence(scores, T, q)
    res = dict(scores=scores, ids=ids, margins=margins, ik=(ikc, iks))
    if attention_tokens is None:
        return res
    use_ids = ids if ids_override is None else ids_override
    tokens = list(attention_tokens)
    # (ids past the context hold no key: the oracle's attention skips them)
    blocks = sorted(set(int(x) for j in tokens for x in use_ids[j].ravel() if 0 <= x and x * BLOCK < T))
    kc = np.zeros((T, 4, 64), np.uint8)
    ks = np.zeros((T, 4, 8), np.uint8)
    vc = np.zeros_like(kc)
    vs = np.zeros_like(ks)
    for blk in blocks:
        t0, t1 = blk * BLOCK, min(T, blk * BLOCK + BLOCK)
        kc[t0:t1], ks[t0:t1] = oracle.quantize(w.kv_rows("k", b, t0, t1).numpy())
        vc[t0:t1], vs[t0:t1] = oracle.quantize(w.kv_rows("v", b, t0, t1).numpy())
    qb = mi.bf16_bits(w.q[b * q:(b + 1) * q])
    sc = oracle.default_scale() if scale is None else scale
    att = np.stack([oracle.sparse_attention_token(qb[j], kc, ks, vc, vs, T, use_ids[j], T - q + j, sc)
                    for j in tokens])
    res["attention"] = att
    res["kv_blocks"] = blocks
    return res


def oracle_rows(w: mi.Workload, b: int, rows: Sequence[int], ids_override: Optional[np.ndarray] = None,
                attention: bool = True):
    """Oracle reference for chosen query tokens j of sequence b, each scored on its own causal
    prefix (tokens 0..p), so that a few rows of a long prefill cost a few prefix scans.
    Returns scores [n][4][max_blocks], ids [n][4][16], margins [n][4] and, if asked,
    attention [n][64][128] over ids_override[n] (else over the oracle's own ids)."""
    import oracle
    T, q = w.ctx_lens[b], w.q_len
    rows = list(rows)
    last = T - q + max(rows) + 1
    ikc, iks = oracle.quantize(w.ik_rows(b, 0, last).numpy())
    qi = mi.bf16_bits(w.q_idx[b * q:(b + 1) * q])
    scores = np.empty((len(rows), 4, w.max_blocks))
    ids = np.empty((len(rows), 4, 16), np.int32)
    margins = np.empty((len(rows), 4))
    for i, j in enumerate(rows):
        p = T - q + j
        scores[i] = oracle.index_scores(qi[j:j + 1], ikc[:p + 1], iks[:p + 1], p + 1, 1, w.max_blocks)[0]
        sid, m = oracle.select_sequence(scores[i:i + 1], p + 1, 1)
        ids[i], margins[i] = sid[0], m[0]
    res = dict(scores=scores, ids=ids, margins=margins, ik=(ikc, iks))
    if not attention:
        return res
    use_ids = ids if ids_override is None else np.asarray(ids_override)
    blocks = sorted(set(int(x) for x in use_ids.ravel() if x >= 0))
    kc = np.zeros((last, 4, 64), np.uint8)
    ks = np.zeros((last, 4, 8), np.uint8)
    vc, vs = np.zeros_like(kc), np.zeros_like(ks)
    for blk in blocks:
        t0, t1 = blk * BLOCK, min(last, blk * BLOCK + BLOCK)
        kc[t0:t1], ks[t0:t1] = oracle.quantize(w.kv_rows("k", b, t0, t1).numpy())
        vc[t0:t1], vs[t0:t1] = oracle.quantize(w.kv_rows("v", b, t0, t1).numpy())
    qb = mi.bf16_bits(w.q[b * q:(b + 1) * q])
    res["attention"] = np.stack([
        oracle.sparse_attention_token(qb[j], kc, ks, vc, vs, last, use_ids[i], T - q + j,
                                      oracle.default_scale()) for i, j in enumerate(rows)])
    return res


def gpu_block_caches(cache, w: mi.Workload, b: int, blocks: Sequence[int]):
    """Logical (codes, scales) of the given blocks of sequence b read back from the GPU pools,
    concatenated in the order given: ik [n*128][64]/[..][8], k and v [n*128][4][64]/[..][4][8]."""
    pages = torch.from_numpy(w.block_table[b, list(blocks)].astype(np.int64))
    out = {}
    ikp = cache.ik[pages.to(cache.ik.device)].cpu().numpy()
    c, s = zip(*[unpack_row_page(pg) for pg in ikp])
    out["ik"] = (np.concatenate(c), np.concatenate(s))
    for name, pool, fn in (("k", cache.k, unpack_row_page), ("v", cache.v, unpack_col_page)):
        pp = pool[pages.to(pool.device)].cpu().numpy()
        cs, ss = [], []
        for pg in pp:
            per_head = [fn(pg[h]) for h in range(4)]
            cs.append(np.stack([x[0] for x in per_head], axis=1))
            ss.append(np.stack([x[1] for x in per_head], axis=1))
        out[name] = (np.concatenate(cs), np.concatenate(ss))
    return out


# ------------------------------------------------------------------ comparisons
def score_tolerance(qi_bits: np.ndarray, ik_codes: np.ndarray, ik_scales: np.ndarray) -> np.ndarray:
    """fp32-accumulation bound per (row): 128 * 2^-24 * ||q|| * max_t ||k_t|| (Cauchy-Schwarz)."""
    import oracle
    keys = oracle.dequantize(ik_codes, ik_scales)
    kmax = float(np.sqrt((keys ** 2).sum(-1)).max()) if len(keys) else 0.0
    qf = (qi_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qn = np.sqrt((qf ** 2).sum(-1))                 # [q][4]
    return 128 * 2.0 ** -24 * qn * kmax + 1e-30


def check_scores(gpu: np.ndarray, ref: np.ndarray, tol: np.ndarray):
    """gpu, ref: [q][4][max_blocks]; tol [q][4]. -inf must match exactly."""
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), "masked blocks differ"
    fin = ~ninf_r
    diff = np.where(fin, np.abs(gpu.astype(np.float64) - np.where(fin, ref, 0)), 0)
    bound = np.broadcast_to(tol[..., None], diff.shape)
    bad = diff > bound
    assert not bad.any(), f"{bad.sum()} scores out of tolerance, worst {diff.max():.3e} (bound {tol.max():.3e})"
    return float(diff.max())


def check_selection(gpu_ids: np.ndarray, ref_ids: np.ndarray, margins: np.ndarray,
                    scores: np.ndarray, tol: np.ndarray, T: int, q: int):
    """Rows with margin >= MARGIN must match exactly; other rows must be a valid selection of
    the oracle scores within the score tolerance. Returns the number of exempt rows."""
    exempt = 0
    for j in range(q):
        n = (T - q + j) // BLOCK + 1
        for g in range(4):
            gi, ri = gpu_ids[j, g], ref_ids[j, g]
            if margins[j, g] >= MARGIN or n <= 16:
                assert np.array_equal(gi, ri), (j, g, gi, ri, margins[j, g])
                continue
            exempt += 1
            sel = gi[gi >= 0]
            assert len(sel) == 16 and len(set(sel.tolist())) == 16 and sel[-1] == n - 1
            assert np.all(np.diff(sel) > 0) and sel.min() >= 0
            s = scores[j, g, :n - 1]
            chosen = np.zeros(n - 1, bool)
            chosen[sel[:-1]] = True
            t = 2 * tol[j, g]
            assert s[chosen].min() >= s[~chosen].max() - t, (j, g)
    return exempt


def check_attention(gpu: np.ndarray, ref: np.ndarray):
    g = gpu.astype(np.float64)
    diff = np.abs(g - ref)
    bad = diff > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{bad.sum()} outputs out of tolerance; worst abs {diff.max():.3e}"
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= REL_L2, f"relative L2 error {rel:.3e}"
    return float(diff.max()), float(rel)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_step_against_oracle(w: mi.Workload, scores: np.ndarray, ids: np.ndarray,
                              att: np.ndarray, max_tokens: int = 8) -> int:
    """A step's block scores, selection and attention outputs (request-major rows) against the
    oracle, sequence by sequence: scores within the fp32 bound, selections bit-exact where the
    margin holds (valid otherwise), attention of up to `max_tokens` query tokens per sequence over
    the GPU's own (validated) selection. Returns the number of rows exempt from the bit compare."""
    q = w.q_len
    exempt_total = 0
    for b in range(w.batch):
        T = w.ctx_lens[b]
        rows = slice(b * q, (b + 1) * q)
        ref = oracle_sequence(w, b)
        tol = score_tolerance(mi.bf16_bits(w.q_idx[rows]), *ref["ik"])
        check_scores(scores[rows], ref["scores"], tol)
        exempt_total += check_selection(ids[rows], ref["ids"], ref["margins"], ref["scores"], tol, T, q)
        toks = list(range(q)) if q <= max_tokens else sorted(set([0, 1, q // 2, q - 2, q - 1]))
        ref = oracle_sequence(w, b, attention_tokens=toks, ids_override=ids[rows])
        check_attention(att[rows][toks], ref["attention"])
    return exempt_total
