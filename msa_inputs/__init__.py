"""Seeded synthetic inputs for the MSA decode workloads.

This module is shared by the tests, the benchmark and the smoke check. It holds no step of the
method (no quantization, scoring, selection or attention): it only draws numbers and lays out
the workload's structure (context lengths, page permutation, block table, planted blocks).

Random numbers
  * Bulk tensors (index keys, K, V, queries) are drawn with a counter-based generator written
    in integer torch ops, so any slice can be regenerated on its own and the CPU and the GPU
    produce the same bits: a 32-bit integer hash of (seed, tag, stream, element index) selects
    an entry of a fixed table of 2^22 draws. The tables are made once from numpy's seeded
    PCG64 generator (standard normal; Student-t with 3 degrees of freedom scaled to unit
    variance), so every value is an exact sample of that distribution and the whole pipeline
    is bit-reproducible on any device.
  * Small structural draws (plant choices and strengths, lengths, permutations) use numpy's
    seeded Generator on the host.

Workloads (shapes of the MiniMax-M3.1 MSA layer: 64 query heads, 4 KV heads, head_dim 128,
one shared 128-d index-key head, 128-token blocks, top-16):
  1 tiny      B=1,  T=4,096,  q=1   N(0,1) data, 16 planted blocks per group (alpha 2),
                                    contiguous page table
  2 batched   B=32, T=32,768, q=1   16 planted blocks per (sequence, group), alpha 2, pool of
                                    8,192 pages in a seeded random permutation
  3 spec128k  B=8,  T=131,072, q=4  4 draft tokens per sequence in the last block; index
                                    queries (u + z)/sqrt(2) share a direction u per
                                    (sequence, group); 16 planted blocks, alpha ~ U[1.5, 3]
  4 ragged    B=6,  T log-uniform in [8K, 512K], never a multiple of 128, q=1; heavy-tailed
                                    index keys (Student-t 3 / sqrt 3), no planting
  5 prefill   B=2,  T=65,536 + 2,048, q=2,048; 15 planted prefix blocks per (sequence, group)
  6 prefix    B=64 requests sharing a 32,768-token prefix (256 blocks: the same pages and the
                                    same data in every sequence), each with a suffix of its own
                                    of log-uniform length in [1K, 8K] tokens (never a multiple of
                                    128), q=1; index queries (u + z)/sqrt(2) share a direction u
                                    per group across the whole batch; 32 planted prefix blocks
                                    per group, the same for every request, alpha ~ U[1.5, 3]
Planting adds alpha * w[b, g] (w = the group's index-query direction) to every index key of a
chosen block, in fp32, before quantization.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

BLOCK = 128
D = 128
KV_HEADS = 4
Q_HEADS = 64
TOPK = 16

POOL_BITS = 22
_MASK32 = 0xFFFFFFFF
_MUL = 0x45D9F3B  # odd multiplier below 2^31: products of 32-bit values stay below 2^63

# tags of the independent random streams
TAG_QI, TAG_Q, TAG_IK, TAG_K, TAG_V, TAG_PLANT, TAG_ALPHA, TAG_PERM, TAG_LEN, TAG_U, TAG_Z, TAG_NEW = range(1, 13)

_pools: Dict[Tuple[str, str], torch.Tensor] = {}


def _pool(kind: str, device) -> torch.Tensor:
    key = (kind, str(device))
    if key not in _pools:
        host_key = (kind, "cpu")
        if host_key not in _pools:
            rng = np.random.default_rng([0x5EED, 1 if kind == "normal" else 2])
            n = 1 << POOL_BITS
            if kind == "normal":
                vals = rng.standard_normal(n, dtype=np.float64)
            elif kind == "t3":
                z = rng.standard_normal(n, dtype=np.float64)
                chi2 = rng.chisquare(3.0, n)
                vals = z / np.sqrt(chi2 / 3.0) / math.sqrt(3.0)
            else:
                raise ValueError(kind)
            _pools[host_key] = torch.from_numpy(vals.astype(np.float32))
        _pools[key] = _pools[host_key].to(device)
    return _pools[key]


def _mix_int(x: int) -> int:
    x &= _MASK32
    for _ in range(2):
        x ^= x >> 16
        x = (x * _MUL) & _MASK32
    x ^= x >> 16
    return x


def _mix(x: torch.Tensor) -> torch.Tensor:
    """The same 32-bit mixer as _mix_int, on int64 tensors holding values in [0, 2^32)."""
    for _ in range(2):
        x = x ^ (x >> 16)
        x = (x * _MUL) & _MASK32
    x = x ^ (x >> 16)
    return x


def stream_key(seed: int, tag: int, *stream: int) -> Tuple[int, int]:
    k = _mix_int(seed * 0x9E3779B1 + tag)
    for s in stream:
        k = _mix_int(k ^ _mix_int(s + 0x632BE5AB))
    return k, _mix_int(k + 0x7F4A7C15)


def draw(kind: str, key: Tuple[int, int], start: int, count: int, device="cpu") -> torch.Tensor:
    """Elements [start, start+count) of the stream `key`, as float32 on `device`."""
    idx = torch.arange(start, start + count, dtype=torch.int64, device=device)
    h = _mix((idx & _MASK32) ^ key[0])
    h = _mix(h ^ ((idx >> 32) * 0x3C6EF372 & _MASK32) ^ key[1])
    return _pool(kind, device)[h >> (32 - POOL_BITS)]


def _host_rng(seed: int, tag: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag, *[int(s) for s in stream]])


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    q_len: int
    ctx_lens: List[int]
    num_pages: int
    block_table: np.ndarray            # int32 [batch][max_blocks], -1 past the sequence
    ik_kind: str                       # "normal" or "t3"
    plants: Dict[Tuple[int, int], List[Tuple[int, float]]]  # (b, g) -> [(block, alpha)]
    plant_dir: np.ndarray              # float32 [batch][4][128]: w[b, g]
    q_idx: torch.Tensor                # bf16 [batch*q][4][128]
    q: torch.Tensor                    # bf16 [batch*q][64][128]
    retries: Dict[int, int]
    prefix_tokens: int = 0             # tokens 0..prefix_tokens-1: sequence 0's, in every sequence

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def n_blocks(self, b: int) -> int:
        return (self.ctx_lens[b] + BLOCK - 1) // BLOCK

    def retry(self, b: int) -> int:
        return int(self.retries.get(b, 0))

    # --------------------------------------------------------------- bulk fp32 data
    def _split_prefix(self, b: int, t0: int, t1: int, rows):
        """Rows [t0, t1) of sequence b when part of them lies in the shared prefix: that part is
        sequence 0's (the same data in every sequence), the rest the sequence's own."""
        mid = min(t1, self.prefix_tokens)
        head = rows(0, t0, mid)
        return head if mid == t1 else torch.cat([head, rows(b, mid, t1)])

    def ik_rows(self, b: int, t0: int, t1: int, device="cpu") -> torch.Tensor:
        """fp32 index keys of sequence b, tokens [t0, t1): noise plus planted directions."""
        if b != 0 and t0 < self.prefix_tokens:
            return self._split_prefix(b, t0, t1, lambda bb, a, z: self.ik_rows(bb, a, z, device))
        key = stream_key(self.seed, TAG_IK, b, self.retry(b))
        x = draw(self.ik_kind, key, t0 * D, (t1 - t0) * D, device).view(t1 - t0, D)
        for g in range(KV_HEADS):
            for blk, alpha in self.plants.get((b, g), []):
                lo, hi = max(t0, blk * BLOCK), min(t1, blk * BLOCK + BLOCK)
                if lo >= hi:
                    continue
                shift = torch.from_numpy(np.float32(alpha) * self.plant_dir[b, g]).to(device)
                x[lo - t0:hi - t0] = x[lo - t0:hi - t0] + shift
        return x

    def kv_rows(self, which: str, b: int, t0: int, t1: int, device="cpu") -> torch.Tensor:
        """fp32 K (which='k') or V (which='v') of sequence b, tokens [t0, t1): [n][4][128]."""
        if b != 0 and t0 < self.prefix_tokens:
            return self._split_prefix(b, t0, t1, lambda bb, a, z: self.kv_rows(which, bb, a, z, device))
        key = stream_key(self.seed, TAG_K if which == "k" else TAG_V, b)
        return draw("normal", key, t0 * KV_HEADS * D, (t1 - t0) * KV_HEADS * D,
                    device).view(t1 - t0, KV_HEADS, D)

    def slots(self, b: int, t0: int, t1: int) -> np.ndarray:
        """Physical slot (page * 128 + offset) of tokens [t0, t1) of sequence b."""
        t = np.arange(t0, t1, dtype=np.int64)
        return self.block_table[b, t // BLOCK].astype(np.int64) * BLOCK + t % BLOCK

    def new_token_rows(self) -> List[Tuple[int, int]]:
        """(sequence, position) of the B*q query tokens, request-major."""
        return [(b, self.ctx_lens[b] - self.q_len + j) for b in range(self.batch) for j in range(self.q_len)]


def _planted_blocks(rng: np.random.Generator, n_choices: int, count: int) -> List[int]:
    return sorted(int(x) for x in rng.choice(n_choices, size=min(count, n_choices), replace=False))


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


CONFIGS = {
    1: dict(name="tiny", batch=1, ctx=4096, q_len=1),
    2: dict(name="batched", batch=32, ctx=32768, q_len=1),
    3: dict(name="spec128k", batch=8, ctx=131072, q_len=4),
    4: dict(name="ragged", batch=6, ctx=None, q_len=1),
    5: dict(name="prefill", batch=2, ctx=65536 + 2048, q_len=2048),
    6: dict(name="prefix", batch=64, ctx=None, q_len=1),
}
PREFIX_BLOCKS = 256  # config 6: the shared prefix


def make_workload(cfg: int, batch: Optional[int] = None, ctx: Optional[int] = None,
                  q_len: Optional[int] = None, ctx_lens: Optional[List[int]] = None,
                  retries: Optional[Dict[int, int]] = None, seed: Optional[int] = None,
                  n_plant: Optional[int] = None, spare_pages: int = 0,
                  prefix_blocks: Optional[int] = None) -> Workload:
    """Build workload `cfg` (1..6) at its stated size, or a reduced variant of the same recipe.

    batch/ctx/q_len/ctx_lens override the sizes; `retries` maps a sequence to the retry counter
    that redraws its index-key noise and plant choices; `seed` defaults to the config number.
    Config 6: `prefix_blocks` sets the shared prefix (default PREFIX_BLOCKS); explicit
    `ctx_lens` must leave every sequence's query tokens past it.
    """
    spec = CONFIGS[cfg]
    seed = cfg if seed is None else seed
    B = spec["batch"] if batch is None else batch
    q = spec["q_len"] if q_len is None else q_len
    retries = dict(retries or {})
    P = (PREFIX_BLOCKS if prefix_blocks is None else prefix_blocks) if cfg == 6 else 0
    if ctx_lens is None:
        if cfg == 6:
            rng = _host_rng(seed, TAG_LEN)
            u = rng.random(B)
            lens = [P * BLOCK + int(round(math.exp(math.log(1024) + x * (math.log(8192) - math.log(1024)))))
                    for x in u]
            ctx_lens = [t - 1 if t % BLOCK == 0 else t for t in lens]
        elif cfg == 4 and ctx is None:
            rng = _host_rng(seed, TAG_LEN)
            u = rng.random(B)
            lens = [int(round(math.exp(math.log(8192) + x * (math.log(524288) - math.log(8192))))) for x in u]
            ctx_lens = [t - 1 if t % BLOCK == 0 else t for t in lens]
        else:
            ctx_lens = [spec["ctx"] if ctx is None else ctx] * B
    ctx_lens = [int(t) for t in ctx_lens]
    assert all(t >= q for t in ctx_lens), "every context must hold its query tokens"
    assert all(t - q >= P * BLOCK for t in ctx_lens), "the shared prefix holds no query token"
    nbs = [(t + BLOCK - 1) // BLOCK for t in ctx_lens]
    max_blocks = max(nbs)
    num_pages = sum(nbs) - (B - 1) * P + spare_pages
    if cfg == 1:
        perm = np.arange(num_pages, dtype=np.int64)
    else:
        perm = _host_rng(seed, TAG_PERM).permutation(num_pages)
    table = np.full((B, max_blocks), -1, np.int32)
    table[:, :P] = perm[:P]  # config 6: every sequence's prefix blocks are the same pages
    off = P
    for b, nb in enumerate(nbs):
        table[b, P:nb] = perm[off:off + nb - P]
        off += nb - P

    # queries
    rows = B * q
    qk = stream_key(seed, TAG_Q)
    Q = _bf16(draw("normal", qk, 0, rows * Q_HEADS * D).view(rows, Q_HEADS, D))
    if cfg == 6:
        # one direction per group for the whole batch
        u = draw("normal", stream_key(seed, TAG_U), 0, KV_HEADS * D).view(1, 1, KV_HEADS, D)
        z = draw("normal", stream_key(seed, TAG_Z), 0, rows * KV_HEADS * D).view(B, q, KV_HEADS, D)
        qi = _bf16(((u + z) * np.float32(1.0 / math.sqrt(2.0))).reshape(rows, KV_HEADS, D))
        plant_dir = u.expand(B, 1, KV_HEADS, D).reshape(B, KV_HEADS, D).numpy().copy()
    elif cfg in (3, 5):
        u = draw("normal", stream_key(seed, TAG_U), 0, B * KV_HEADS * D).view(B, 1, KV_HEADS, D)
        z = draw("normal", stream_key(seed, TAG_Z), 0, rows * KV_HEADS * D).view(B, q, KV_HEADS, D)
        qi = _bf16(((u + z) * np.float32(1.0 / math.sqrt(2.0))).reshape(rows, KV_HEADS, D))
        plant_dir = u.reshape(B, KV_HEADS, D).numpy().copy()
    else:
        qi = _bf16(draw("normal", stream_key(seed, TAG_QI), 0, rows * KV_HEADS * D).view(rows, KV_HEADS, D))
        # w[b, g] = the fp32 value of the group's (first) index query
        plant_dir = qi.view(B, q, KV_HEADS, D)[:, 0].float().numpy().copy()

    plants: Dict[Tuple[int, int], List[Tuple[int, float]]] = {}
    if cfg == 6:
        # planted prefix blocks, the same for every request (they live in the shared data)
        count = 32 if n_plant is None else n_plant
        for g in range(KV_HEADS):
            blocks = _planted_blocks(_host_rng(seed, TAG_PLANT, 0, g, retries.get(0, 0)), P, count)
            arng = _host_rng(seed, TAG_ALPHA, 0, g, retries.get(0, 0))
            alphas = [float(np.float32(a)) for a in arng.uniform(1.5, 3.0, len(blocks))]
            for b in range(B):
                plants[(b, g)] = list(zip(blocks, alphas))
    elif cfg != 4:
        count = {1: 16, 2: 16, 3: 16, 5: 15}[cfg] if n_plant is None else n_plant
        for b in range(B):
            r = retries.get(b, 0)
            # config 5 plants only in the cached prefix (blocks before the chunk)
            n_choices = nbs[b] if cfg != 5 else max(1, (ctx_lens[b] - q) // BLOCK)
            for g in range(KV_HEADS):
                rng = _host_rng(seed, TAG_PLANT, b, g, r)
                blocks = _planted_blocks(rng, n_choices, count)
                if cfg == 3:
                    arng = _host_rng(seed, TAG_ALPHA, b, g, r)
                    alphas = [float(np.float32(a)) for a in arng.uniform(1.5, 3.0, len(blocks))]
                else:
                    alphas = [2.0] * len(blocks)
                plants[(b, g)] = list(zip(blocks, alphas))
    return Workload(name=spec["name"], seed=seed, batch=B, q_len=q, ctx_lens=ctx_lens,
                    num_pages=num_pages, block_table=table,
                    ik_kind="t3" if cfg == 4 else "normal", plants=plants,
                    plant_dir=plant_dir.astype(np.float32), q_idx=qi.contiguous(), q=Q.contiguous(),
                    retries=retries, prefix_tokens=P * BLOCK)


RETRIES_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tests", "golden", "retries.json")


def full_workload(cfg: int) -> Workload:
    """Workload `cfg` at its stated size, with the margin-enforcing retry counters that
    tests/golden/make_retries.py found with the oracle (every selection row then has a margin
    of at least 1e-3). Without that file, every counter is 0."""
    retries = {}
    if os.path.exists(RETRIES_FILE):
        with open(RETRIES_FILE) as f:
            doc = json.load(f)
        retries = {int(b): int(r) for b, r in doc.get(str(cfg), {}).get("retries", {}).items()}
    return make_workload(cfg, retries=retries)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (CPU numpy)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
