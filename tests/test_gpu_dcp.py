"""Block selection split over shards and merged (indexer context parallelism on one device),
bit for bit against the oracle and against the single-call selection (needs an MI355X).

"vLLM day-0 support for MiniMax-M3.1-Flash", section "Indexer NVFP4 DCP": each device keeps a
local top 16 per index head over its share of the pages; the owner merges the lists into the
final top 16, and the selection stays exact. Shards here are contiguous slices with random cuts
(passed as column views of the full score tensor) and the round-robin split (block i on shard
i % N, passed as compact per-shard score tensors), over 2 to 8 shards, on the constructed score
rows of the selection tests (ties, signed zeros, -inf) and on rows with 0 to max_blocks eligible
blocks, for shards held as 16 and as 64 keys per lane.
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_selection import _patterns

pytestmark = pytest.mark.gpu

Q_LEN = 3


def _rank_key(x: np.float32) -> int:
    """The rank key the header defines: order-preserving bits of the fp32 score, -0 as +0."""
    u = int(np.array([x + np.float32(0.0)], np.float32).view(np.uint32)[0])
    return (u ^ 0x80000000) if u < 0x80000000 else (~u & 0xFFFFFFFF)


def _shards(kind, n_shards, max_blocks, rng):
    if kind == "contiguous":
        cuts = np.sort(rng.choice(np.arange(1, max_blocks), size=n_shards - 1, replace=False))
        bounds = [0, *cuts.tolist(), max_blocks]
        return [(lo, 1, hi - lo) for lo, hi in zip(bounds[:-1], bounds[1:])]
    return [(s, n_shards, len(range(s, max_blocks, n_shards))) for s in range(n_shards)]


@pytest.mark.parametrize("max_blocks,n_shards,kind", [
    (1024, 2, "contiguous"), (1024, 3, "round_robin"), (1024, 4, "contiguous"),
    (1024, 4, "round_robin"), (1024, 8, "contiguous"), (2048, 2, "round_robin"),
    (2048, 8, "round_robin"), (4097, 2, "contiguous"), (4097, 4, "round_robin"),
])
def test_shard_merge_matches_single_selection(max_blocks, n_shards, kind):
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(1000 * n_shards + max_blocks + (kind == "contiguous"))
    pats = _patterns(max_blocks, rng)
    mb = max_blocks
    # context lengths: rows with no eligible block (p < 0), 1, 16, 17, 18, 65, and full rows
    ctx = [1, 16 * 128 + 1, 18 * 128, 65 * 128, 128 * (mb - 1) + 1, 128 * mb]
    batch = len(ctx)
    rows = batch * Q_LEN
    scores = np.stack([pats[(r * 3 + g) % len(pats)] for r in range(rows) for g in range(4)])
    scores = scores.reshape(rows, 4, mb).astype(np.float32)
    ns = [[0 if (p := T - Q_LEN + j) < 0 else min(p // 128 + 1, mb) for j in range(Q_LEN)] for T in ctx]

    b = msa.Batch(torch.zeros((batch, mb), dtype=torch.int32, device="cuda"),
                  torch.tensor(ctx, dtype=torch.int32, device="cuda"), Q_LEN)
    s_dev = torch.from_numpy(scores).cuda()
    shards = _shards(kind, n_shards, mb, rng)
    cand_ids = torch.full((n_shards, rows, 4, 16), -7, dtype=torch.int32, device="cuda")
    cand_keys = torch.full((n_shards, rows, 4, 16), 7, dtype=torch.int32, device="cuda")
    for s, (begin, stride, n_cols) in enumerate(shards):
        if stride == 1:
            view = s_dev[:, :, begin:begin + n_cols]  # a column slice: row stride max_blocks
        else:
            view = s_dev[:, :, begin::stride].contiguous()
        assert view.shape[2] == n_cols
        msa.msa_block_topk_local(view, begin, stride, b, 16, cand_ids[s], cand_keys[s])
    merged = torch.full((rows, 4, 16), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk_merge(cand_ids, cand_keys, b, 16, merged)
    direct = torch.full((rows, 4, 16), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk(s_dev, b, 16, direct)
    torch.cuda.synchronize()

    got_ids = cand_ids.cpu().numpy()
    got_keys = cand_keys.cpu().numpy().view(np.uint32)
    got_merged = merged.cpu().numpy()
    assert np.array_equal(got_merged, direct.cpu().numpy())
    for i in range(batch):
        for j in range(Q_LEN):
            r, n = i * Q_LEN + j, ns[i][j]
            for g in range(4):
                row = scores[r, g]
                lists = []
                for s, (begin, stride, n_cols) in enumerate(shards):
                    want, forced = oracle.dcp_local_topk(row.astype(np.float64), n,
                                                         range(begin, begin + stride * n_cols, stride))
                    lists.append(want)
                    pad = 16 - len(want)
                    assert list(got_ids[s, r, g]) == want + [-1] * pad, (s, r, g, n)
                    want_keys = [0xFFFFFFFF if f else _rank_key(row[k]) for k, f in zip(want, forced)]
                    assert list(got_keys[s, r, g]) == want_keys + [0] * pad, (s, r, g, n)
                ref = oracle.dcp_merge(row.astype(np.float64), n, lists)
                assert list(got_merged[r, g]) == list(ref), (r, g, n)
                single, _ = oracle.block_topk(row.astype(np.float64), n)
                assert list(ref) == list(single)


def test_merge_of_one_shard_and_of_padded_lists():
    # one shard holding every block merges to itself; a second shard with only padding changes
    # nothing
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(77)
    mb, ctx = 300, [300 * 128, 40 * 128 + 5, 7 * 128]
    batch = len(ctx)
    scores = np.round(rng.standard_normal((batch * Q_LEN, 4, mb)) * 3).astype(np.float32)
    b = msa.Batch(torch.zeros((batch, mb), dtype=torch.int32, device="cuda"),
                  torch.tensor(ctx, dtype=torch.int32, device="cuda"), Q_LEN)
    s_dev = torch.from_numpy(scores).cuda()
    cand_ids = torch.full((2, batch * Q_LEN, 4, 16), -1, dtype=torch.int32, device="cuda")
    cand_keys = torch.zeros((2, batch * Q_LEN, 4, 16), dtype=torch.int32, device="cuda")
    msa.msa_block_topk_local(s_dev, 0, 1, b, 16, cand_ids[0], cand_keys[0])
    direct = torch.empty((batch * Q_LEN, 4, 16), dtype=torch.int32, device="cuda")
    msa.msa_block_topk(s_dev, b, 16, direct)
    one = torch.empty_like(direct)
    msa.msa_block_topk_merge(cand_ids[:1].contiguous(), cand_keys[:1].contiguous(), b, 16, one)
    two = torch.empty_like(direct)
    msa.msa_block_topk_merge(cand_ids, cand_keys, b, 16, two)
    torch.cuda.synchronize()
    d = direct.cpu().numpy()
    assert np.array_equal(cand_ids[0].cpu().numpy(), d)  # the local list of the whole row
    assert np.array_equal(one.cpu().numpy(), d)
    assert np.array_equal(two.cpu().numpy(), d)
