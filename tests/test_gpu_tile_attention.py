"""Attention over given block ids that differ from token to token, in the launch shape that
takes the token-tile kernel (8+ query tokens per sequence, 1,024+ rows), against the oracle
(needs an MI355X).

The selections here are random rather than from the indexer, so the 16 tokens of a tile
(two per wavefront) share few blocks and their union reaches past 128 entries. They also
include blocks past a token's position (skipped for that token, still in the union for the
others), -1 padding, and rows left with no block at all (output 0). "vLLM day-0 support
for MiniMax-M3.1-Flash", section "MSA primer": exact attention over the selected blocks only;
"MiniMax M3 on vLLM", section "Prefill execution": per-token causal positions.
"""
import numpy as np
import pytest
import torch

import msa_inputs as mi
from msa_testlib import DeviceWorkload, bf16_to_f64, check_attention, oracle_rows

pytestmark = pytest.mark.gpu

Q_LEN = 32


def _random_ids(w, rng):
    """ids [batch * q][4][16]: mostly distinct random blocks at or below the token's block,
    some past it, some -1; ascending with -1 last, as the selection writes them."""
    B, q = w.batch, w.q_len
    ids = np.full((B * q, 4, 16), -1, np.int32)
    for b in range(B):
        T = w.ctx_lens[b]
        nb_ctx = (T + 127) // 128
        for j in range(q):
            p = T - q + j
            n_elig = p // 128 + 1
            for g in range(4):
                kind = rng.integers(0, 10)
                if kind == 0:
                    continue  # no block: output 0
                k = 16 if b % 2 else int(rng.integers(1, 17))
                pool = np.arange(nb_ctx)  # includes blocks past p when the context has them
                pick = rng.choice(pool, size=min(k, len(pool)), replace=False)
                if kind == 1:
                    pick = pick[pick >= n_elig][:3]  # only future blocks: nothing visible
                pick = np.sort(pick)
                ids[b * q + j, g, :len(pick)] = pick
    return ids


def test_tile_attention_random_selections():
    w = mi.make_workload(3, batch=8, ctx_lens=[3000, 20000, 9000, 30000, 4100, 25000, 8200, 2500],
                         q_len=Q_LEN)
    assert w.batch * w.q_len * 4 >= 1024  # the token-tile launch shape
    g = DeviceWorkload(w)
    g.run()
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(11)
    ids = _random_ids(w, rng)
    # union sizes of the tiles of 16 tokens (this test's point: past 128 entries for some)
    unions = [len({int(x) for x in ids[b * Q_LEN + t0:b * Q_LEN + t0 + 16, gg].ravel() if x >= 0})
              for b in range(w.batch) for t0 in range(0, Q_LEN, 16) for gg in range(4)]
    assert max(unions) > 128
    ids_dev = torch.from_numpy(ids).cuda()
    out = torch.full_like(g.step.out, 7.0)
    msa.msa_sparse_attn_decode(g.cache, g.batch, g.q, ids_dev, msa.default_softmax_scale(), out,
                               g.step.workspace)
    torch.cuda.synchronize()
    att = bf16_to_f64(out)
    rows = [0, 5, 8, 15, 23, 31]
    for b in range(w.batch):
        sel = ids[b * Q_LEN:(b + 1) * Q_LEN][rows]
        ref = oracle_rows(w, b, rows, ids_override=sel)
        check_attention(att[b * Q_LEN:(b + 1) * Q_LEN][rows], ref["attention"])
        for i, j in enumerate(rows):
            for gg in range(4):
                if not (sel[i, gg] >= 0).any():
                    assert np.all(att[b * Q_LEN + j, 16 * gg:16 * gg + 16] == 0.0), (b, j, gg)
