"""Block selection on constructed score rows, bit for bit against the oracle (needs an MI355X).

Rows that stress the selection's bound, compaction and tie paths: all scores equal (every
candidate reaches the bound, the counted-extraction path), more than 64 blocks tied at the top,
exactly 15 distinct leaders over a flat rest, a tie of 70 blocks at the 15th place, signed
zeros, -inf scores, and plain random rows; at several row lengths (eligible block counts from
the trivial 16 to full rows) and for rows held as 16 and as 64 keys per lane; both through the
selection kernel and through the selection inside the attention launch (its ids output).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _patterns(n_blocks, rng):
    out = []
    out.append(np.zeros(n_blocks, np.float32))
    out.append(np.where(rng.random(n_blocks) < 0.5, -0.0, 0.0).astype(np.float32))
    x = rng.standard_normal(n_blocks).astype(np.float32)
    x[rng.choice(n_blocks, min(100, n_blocks), replace=False)] = 9.0
    out.append(x)
    x = np.full(n_blocks, -1.0, np.float32)
    lead = rng.choice(n_blocks, min(15, n_blocks), replace=False)
    x[lead] = np.arange(len(lead), dtype=np.float32) + 2.0
    out.append(x)
    x = rng.standard_normal(n_blocks).astype(np.float32) - 10.0
    top = rng.choice(n_blocks, min(84, n_blocks), replace=False)
    x[top[:14]] = np.arange(14, dtype=np.float32) + 5.0
    x[top[14:]] = 3.0
    out.append(x)
    x = rng.standard_normal(n_blocks).astype(np.float32)
    x[rng.random(n_blocks) < 0.3] = -np.inf
    out.append(x)
    out.append(rng.standard_normal(n_blocks).astype(np.float32))
    out.append(np.round(rng.standard_normal(n_blocks) * 4.0).astype(np.float32))
    return out


@pytest.mark.parametrize("max_blocks", [1024, 2048])
def test_selection_constructed_rows(max_blocks):
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(5 + max_blocks)
    pats = _patterns(max_blocks, rng)
    # eligible block counts: the query token of sequence b sits in block n_b - 1
    n_list = [16, 17, 18, 63, 64, 65, 129, max_blocks - 1, max_blocks]
    rows, ns = [], []
    for n in n_list:
        for g in range(4):
            rows.append(pats[(len(ns) + g) % len(pats)])
        ns.append(n)
    batch = len(n_list)
    scores = np.stack(rows).reshape(batch, 4, max_blocks).astype(np.float32)
    ctx = torch.tensor([128 * (n - 1) + 1 for n in ns], dtype=torch.int32, device="cuda")
    table = torch.zeros((batch, max_blocks), dtype=torch.int32, device="cuda")
    b = msa.Batch(table, ctx, 1)
    ids = torch.empty((batch, 4, 16), dtype=torch.int32, device="cuda")
    s_dev = torch.from_numpy(scores).cuda()
    msa.msa_block_topk(s_dev, b, 16, ids)
    results = {"topk": ids}
    if max_blocks <= 1024:
        # the attention launch that selects for itself (an all-zero one-page cache: only its ids
        # output is checked here)
        cache = msa.Cache.allocate(1)
        q = torch.zeros((batch, 64, 128), dtype=torch.bfloat16, device="cuda")
        out = torch.empty_like(q)
        ws_bytes = msa.msa_sparse_attn_workspace_bytes(b)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
        ids2 = torch.full((batch, 4, 16), -7, dtype=torch.int32, device="cuda")
        msa.msa_select_attn_decode(cache, b, s_dev, 16, ids2, q, 0.088, out, ws)
        results["select_attention"] = ids2
    torch.cuda.synchronize()
    for path, t in results.items():
        got = t.cpu().numpy()
        for i, n in enumerate(ns):
            for g in range(4):
                want, _ = oracle.block_topk(scores[i, g].astype(np.float64), n)
                assert np.array_equal(got[i, g], want), (path, max_blocks, n, g, got[i, g], want)


@pytest.mark.parametrize("max_blocks", [1024, 2048])
@pytest.mark.parametrize("topk,init,local", [(16, 0, 1), (16, 2, 3), (8, 1, 1), (32, 0, 4),
                                             (64, 4, 2), (16, 0, 0), (5, 3, 2)])
def test_window_selection_constructed_rows(max_blocks, topk, init, local):
    # the window knobs ("MiniMax M3 on vLLM", section "MSA mechanism": init and local blocks),
    # bit for bit against the oracle; (16, 0, 1) is the recipe and must equal msa_block_topk
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(7 + max_blocks + 100 * topk + 10 * init + local)
    pats = _patterns(max_blocks, rng)
    n_list = [1, 5, topk, topk + 1, topk + 2, 63, 64, 65, 129, max_blocks - 1, max_blocks]
    rows = []
    for i in range(len(n_list)):
        for g in range(4):
            rows.append(pats[(i + g) % len(pats)])
    batch = len(n_list)
    scores = np.stack(rows).reshape(batch, 4, max_blocks).astype(np.float32)
    ctx = torch.tensor([128 * (n - 1) + 1 for n in n_list], dtype=torch.int32, device="cuda")
    b = msa.Batch(torch.zeros((batch, max_blocks), dtype=torch.int32, device="cuda"), ctx, 1)
    s_dev = torch.from_numpy(scores).cuda()
    ids = torch.full((batch, 4, topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk_window(s_dev, b, topk, init, local, ids)
    direct = None
    if (topk, init, local) == (16, 0, 1):
        direct = torch.full((batch, 4, 16), -7, dtype=torch.int32, device="cuda")
        msa.msa_block_topk(s_dev, b, 16, direct)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for i, n in enumerate(n_list):
        for g in range(4):
            want = oracle.block_topk_variant(scores[i, g].astype(np.float64), n, topk, init, local)
            assert list(got[i, g]) == list(want), (n, g, list(got[i, g]), list(want))
    if direct is not None:
        assert np.array_equal(direct.cpu().numpy(), got)
