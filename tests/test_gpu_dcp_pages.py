"""Indexer context parallelism end to end on one device, from the pages: each shard's pool holds
only its own index-key pages, the indexer scores the shard under global block ids
(msa_indexer_score_shard), msa_block_topk_local keeps its local top 16 and msa_block_topk_merge
merges the shards' lists (needs an MI355X).

"vLLM day-0 support for MiniMax-M3.1-Flash", section "Indexer NVFP4 DCP": each device scores
every index head on its share of the context, the scores are bit for bit those of one device,
and the owner's selection from the merged lists is exact. Checked here: every shard's scores
equal the matching columns of msa_indexer_score on the whole table, bit for bit, and the merged
selection equals msa_block_topk on the whole scores, for 2, 4 and 8 shards cut contiguously (at
seeded random points) and round-robin, on ragged contexts (one ends 5 tokens into its last
block, one is shorter than a shard), with the decode indexer (4 query tokens) and the score-GEMM
indexer (12 query tokens).
"""
import numpy as np
import pytest
import torch

import msa_inputs as mi
from msa_testlib import DeviceWorkload

pytestmark = pytest.mark.gpu

CTX = [21_000, 128 * 41 + 5, 300]


def _shards(kind, n_shards, max_blocks, rng):
    """(begin, stride, n_cols) of each shard."""
    if kind == "contiguous":
        cuts = np.sort(rng.choice(np.arange(1, max_blocks), size=n_shards - 1, replace=False))
        bounds = [0, *cuts.tolist(), max_blocks]
        return [(lo, 1, hi - lo) for lo, hi in zip(bounds[:-1], bounds[1:])]
    return [(s, n_shards, len(range(s, max_blocks, n_shards))) for s in range(n_shards)]


def _shard_cache(msa, cache, table, cols):
    """A pool holding only the index-key pages of the shard's columns, and the shard's table of
    local page ids (-1 where the whole table has none)."""
    sub = table[:, cols]
    pages = np.unique(sub[sub >= 0])
    local = np.full(int(table.max()) + 1, -1, np.int32)
    local[pages] = np.arange(len(pages), dtype=np.int32)
    shard_table = np.ascontiguousarray(np.where(sub >= 0, local[np.maximum(sub, 0)], -1), np.int32)
    sc = msa.Cache.allocate(max(1, len(pages)))
    sc.ik.fill_(0xFF)  # bytes no page copy writes: NaN scales, which must never be read
    if len(pages):
        src = cache.ik.view(-1, 9216)[torch.from_numpy(pages).long().cuda()]
        sc.ik.view(-1, 9216)[: len(pages)].copy_(src)
    return sc, shard_table


@pytest.fixture(scope="module", params=[4, 12], ids=["decode_q4", "gemm_q12"])
def loaded(request):
    import block_sparse_attention_nvfp4_amd as msa
    w = mi.make_workload(3, batch=len(CTX), q_len=request.param, ctx_lens=CTX, seed=41)
    d = DeviceWorkload(w)
    msa.msa_kv_insert_nvfp4(d.cache, d.new_slots, d.new_k, d.new_v, d.new_ik)
    full = torch.empty((w.batch * w.q_len, 4, w.max_blocks), dtype=torch.float32, device="cuda")
    msa.msa_indexer_score(d.cache, d.batch, d.q_idx, full)
    direct = torch.full((w.batch * w.q_len, 4, 16), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk(full, d.batch, 16, direct)
    torch.cuda.synchronize()
    return w, d, full, direct


@pytest.mark.parametrize("n_shards", [2, 4, 8])
@pytest.mark.parametrize("kind", ["contiguous", "round_robin"])
def test_shards_scored_from_their_pages_merge_to_the_single_selection(loaded, kind, n_shards):
    import block_sparse_attention_nvfp4_amd as msa
    w, d, full, direct = loaded
    rows, mb = w.batch * w.q_len, w.max_blocks
    rng = np.random.default_rng(97 * n_shards + (kind == "contiguous"))
    shards = _shards(kind, n_shards, mb, rng)
    cand_ids = torch.full((n_shards, rows, 4, 16), -7, dtype=torch.int32, device="cuda")
    cand_keys = torch.full((n_shards, rows, 4, 16), 7, dtype=torch.int32, device="cuda")
    full_h = full.cpu().numpy()
    for s, (begin, stride, n_cols) in enumerate(shards):
        cols = list(range(begin, begin + stride * n_cols, stride))
        sc, st = _shard_cache(msa, d.cache, w.block_table, cols)
        sb = msa.Batch(torch.from_numpy(st).cuda(), d.ctx, w.q_len)
        got = torch.full((rows, 4, n_cols), 7.0, dtype=torch.float32, device="cuda")
        msa.msa_indexer_score_shard(sc, sb, begin, stride, mb, d.q_idx, got)
        msa.msa_block_topk_local(got, begin, stride, d.batch, 16, cand_ids[s], cand_keys[s])
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        want = full_h[:, :, cols]
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32)), (s, begin, stride)
    merged = torch.full((rows, 4, 16), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk_merge(cand_ids, cand_keys, d.batch, 16, merged)
    torch.cuda.synchronize()
    assert np.array_equal(merged.cpu().numpy(), direct.cpu().numpy())


def test_shard_of_blocks_past_every_context(loaded):
    # a shard whose blocks lie past a short sequence's context scores -inf there, loads nothing
    # for it, and the columns of the long sequence still match
    import block_sparse_attention_nvfp4_amd as msa
    w, d, full, _ = loaded
    rows, mb = w.batch * w.q_len, w.max_blocks
    begin, n_cols = mb - 20, 20
    cols = list(range(begin, mb))
    sc, st = _shard_cache(msa, d.cache, w.block_table, cols)
    sb = msa.Batch(torch.from_numpy(st).cuda(), d.ctx, w.q_len)
    got = torch.full((rows, 4, n_cols), 7.0, dtype=torch.float32, device="cuda")
    msa.msa_indexer_score_shard(sc, sb, begin, 1, mb, d.q_idx, got)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), full.cpu().numpy()[:, :, cols].view(np.uint32))
    assert np.all(g[w.q_len:] == -np.inf)  # sequences 1 and 2 end before block mb - 20
