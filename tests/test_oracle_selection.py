"""Pins of the oracle's indexer (scores + block max-pool) and block selection.

Sources: "vLLM day-0 support for MiniMax-M3.1-Flash", sections "MSA primer" (index score per
key with one index query per GQA group against one shared index-key head; max-pool per 128-token
block; top 16 blocks with the most recent always kept; at most 2,048 keys) and "Indexer NVFP4
DCP" (each device selects a local top-16 over its share of the pages, the owner merges them,
and the merged selection equals the single-device one); "MiniMax M3 on vLLM", section "MSA
mechanism" (local_blocks = 1, init_blocks = 0, partial last block masked, causal boundary
inside a block, the local block not counted twice).
"""
import math

import numpy as np
import pytest

import oracle


def ref_select(scores, n, topk=16):
    """Independent restatement by full sort: forced last block + best topk-1 of the rest."""
    if n <= topk:
        return list(range(n))
    rest = sorted(range(n - 1), key=lambda i: (-scores[i], i))[:topk - 1]
    return sorted(rest + [n - 1])


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_full_sort_small(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 41))
    # few distinct values so ties are frequent
    scores = rng.integers(-5, 6, n).astype(np.float64) * (0.5 if seed % 2 else 1.0)
    ids, margin = oracle.block_topk(scores, n)
    want = ref_select(list(scores), n)
    assert list(ids[:len(want)]) == want
    assert all(x == -1 for x in ids[len(want):])
    if n <= 16:
        assert margin == math.inf


def test_forced_block_kept_even_when_lowest():
    n = 40
    scores = np.arange(n, 0, -1, dtype=np.float64)   # block n-1 has the lowest score
    ids, _ = oracle.block_topk(scores, n)
    assert ids[-1] == n - 1 and list(ids[:15]) == list(range(15))
    assert len(set(ids.tolist())) == 16              # forced block not double-counted


def test_forced_block_not_double_counted_when_also_best():
    n = 30
    scores = np.zeros(n)
    scores[n - 1] = 100.0
    scores[:20] = np.arange(20, 0, -1)
    ids, _ = oracle.block_topk(scores, n)
    assert list(ids) == list(range(15)) + [n - 1]


def test_cap_of_2048_keys():
    scores = np.random.default_rng(0).standard_normal(1000)
    ids, _ = oracle.block_topk(scores, 1000)
    assert (ids >= 0).sum() * 128 == 2048


def test_margin_definition():
    scores = np.array([10.0, 9.0, 8.0] + [1.0] * 14 + [0.5, 0.0])  # n = 19
    ids, margin = oracle.block_topk(scores, 19)
    # kept: blocks 0..14 (scores 10,9,8,1 x12) and 18 (forced); dropped best: 1.0
    assert margin == 0.0
    scores = np.array([float(20 - i) for i in range(18)] + [-3.0])
    ids, margin = oracle.block_topk(scores, 19)
    assert list(ids) == list(range(15)) + [18]
    assert margin == pytest.approx((6.0 - 5.0) / 6.0)


@pytest.mark.parametrize("shards", [2, 3, 4, 8])
def test_dcp_shard_merge_is_exact(shards):
    rng = np.random.default_rng(shards)
    for trial in range(50):
        n = int(rng.integers(17, 300))
        scores = np.round(rng.standard_normal(n), 1)  # ties on purpose
        want, _ = oracle.block_topk(scores, n)
        # each shard takes a contiguous slice of pages and keeps its local best 16 candidates,
        # with the forced block ranked first on the shard that holds it
        cuts = np.sort(rng.choice(np.arange(1, n), size=shards - 1, replace=False))
        bounds = [0, *cuts.tolist(), n]
        cands = []
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            local = sorted(range(lo, hi), key=lambda i: (-(math.inf if i == n - 1 else scores[i]), i))[:16]
            cands += local
        merged = sorted(cands, key=lambda i: (-(math.inf if i == n - 1 else scores[i]), i))[:16]
        assert sorted(merged) == list(want)


def _dequant_keys(codes, scales):
    return oracle.dequantize(codes, scales)


def _bf16_bits(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_float(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("T,q", [(1, 1), (127, 1), (128, 1), (129, 1), (700, 1), (1000, 4), (515, 3)])
def test_index_scores_vs_numpy_bruteforce(T, q):
    rng = np.random.default_rng(T * 7 + q)
    ik = rng.standard_normal((T, 128)).astype(np.float32)
    codes, scales = oracle.quantize(ik)
    qb = _bf16_bits(rng.standard_normal((q, 4, 128)))
    nb = (T + 127) // 128 + 2                       # extra blocks past the end must be -inf
    got = oracle.index_scores(qb, codes, scales, T, q, nb)
    keys = _dequant_keys(codes, scales)             # [T][128]
    tok = keys @ _bits_to_float(qb).reshape(q * 4, 128).T   # [T][q*4]
    for j in range(q):
        p = T - q + j
        for g in range(4):
            for blk in range(nb):
                lo, hi = blk * 128, min(blk * 128 + 128, p + 1)
                want = tok[lo:hi, j * 4 + g].max() if hi > lo else -np.inf
                assert got[j, g, blk] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_index_scores_planted_closed_form():
    # keys that quantize exactly (E2M1 grid values times a power of two) make the score exact
    T = 384
    w = np.array([1.0, -0.5, 6.0, 0.0] * 32, np.float32)   # amax 6 per group: scale 1
    ik = np.zeros((T, 128), np.float32)
    ik[128:256] = 3.0 * w / 2.0                    # block 1 planted with alpha = 1.5
    ik[300] = w                                    # a single token in block 2
    codes, scales = oracle.quantize(ik)
    assert np.array_equal(oracle.dequantize(codes, scales), ik.astype(np.float64))
    qv = np.tile(np.array([0.5, 1.0, 0.25, 3.0], np.float32), 32)
    qb = _bf16_bits(np.tile(qv, (1, 4, 1)))
    got = oracle.index_scores(qb, codes, scales, T, 1, 3)
    dot = float(np.dot(w.astype(np.float64), qv.astype(np.float64)))
    assert np.all(got[0, :, 0] == 0.0)
    assert np.all(got[0, :, 1] == 1.5 * dot)
    assert np.all(got[0, :, 2] == max(dot, 0.0))


def test_causal_mask_inside_last_block():
    # q = 4 draft tokens in the last block: token j sees keys up to T - 4 + j only
    T, q = 256, 4
    ik = np.zeros((T, 128), np.float32)
    ik[T - 1] = 1.5                                 # only the very last key is non-zero (exact)
    codes, scales = oracle.quantize(ik)
    qb = _bf16_bits(np.ones((q, 4, 128)))
    got = oracle.index_scores(qb, codes, scales, T, q, 2)
    assert list(got[:, 0, 1]) == [0.0, 0.0, 0.0, 192.0]
