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


@pytest.mark.parametrize("seed", range(20))
def test_variant_default_knobs_are_the_recipe(seed):
    # init_blocks = 0, local_blocks = 1 is the current recipe: the C oracle's selection, which
    # the full-sort pins above fix independently
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 200))
    scores = np.round(rng.standard_normal(n), 1)
    want, _ = oracle.block_topk(scores, n)
    assert list(oracle.block_topk_variant(scores, n, 16, 0, 1)) == list(want)


def test_variant_by_hand():
    # n = 12 eligible blocks, scores rising with the id except two planted highs
    scores = np.arange(12, dtype=np.float64)
    scores[[2, 5]] = [100.0, 50.0]
    # topk 6, init 2, local 2: forced {0, 1, 10, 11}, then the best two others: 2 (100), 5 (50)
    assert list(oracle.block_topk_variant(scores, 12, 6, 2, 2)) == [0, 1, 2, 5, 10, 11]
    # no forced block at all: the plain top 4 (ties none): 2, 5, 11, 10
    assert list(oracle.block_topk_variant(scores, 12, 4, 0, 0)) == [2, 5, 10, 11]
    # init and local overlap when they reach each other: topk 5, init 3, local 2 -> 0, 1, 2,
    # 10, 11 and nothing else
    assert list(oracle.block_topk_variant(scores, 12, 5, 3, 2)) == [0, 1, 2, 10, 11]
    # at most topk eligible blocks: all of them, padded
    assert list(oracle.block_topk_variant(scores, 3, 4, 1, 1)) == [0, 1, 2, -1]
    # ties at the boundary go to the lower id
    flat = np.zeros(10)
    assert list(oracle.block_topk_variant(flat, 10, 5, 1, 1)) == [0, 1, 2, 3, 9]


@pytest.mark.parametrize("seed", range(30))
def test_variant_brute_force_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 120))
    topk = int(rng.choice([4, 8, 16, 32]))
    init = int(rng.integers(0, topk // 2 + 1))
    local = int(rng.integers(0, topk - init + 1))
    scores = rng.integers(-3, 4, n).astype(np.float64)  # many ties
    got = [int(x) for x in oracle.block_topk_variant(scores, n, topk, init, local) if x >= 0]
    assert got == sorted(set(got)) and len(got) == min(n, topk)
    if n <= topk:
        return
    forced = set(range(min(init, n))) | set(range(max(n - local, 0), n))
    assert forced <= set(got)
    free_kept = [i for i in got if i not in forced]
    dropped = [i for i in range(n) if i not in got]
    # every free kept block ranks before every dropped one by (score desc, id asc)
    for i in free_kept:
        for d in dropped:
            assert (scores[i], -i) > (scores[d], -d)


def _shard_splits(rng, n, shards):
    """Contiguous slices with random cuts, and the round-robin split (block i on shard i % N)."""
    cuts = np.sort(rng.choice(np.arange(1, n), size=shards - 1, replace=False))
    bounds = [0, *cuts.tolist(), n]
    contiguous = [range(lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]
    round_robin = [range(s, n, shards) for s in range(shards)]
    return contiguous, round_robin


@pytest.mark.parametrize("shards", [2, 3, 4, 8])
def test_dcp_shard_merge_is_exact(shards):
    # the merged local lists equal the single-device selection, which the full-sort pins above
    # fix independently; ties on purpose, and rows of up to 16 eligible blocks (all kept)
    rng = np.random.default_rng(shards)
    for trial in range(60):
        n = int(rng.integers(max(shards, 2), 300)) if trial % 4 else int(rng.integers(max(shards, 2), 17))
        scores = np.round(rng.standard_normal(n + 5), 1)
        want, _ = oracle.block_topk(scores, n)
        ref = ref_select(scores, n)
        assert list(want) == ref + [-1] * (16 - len(ref))
        for split in _shard_splits(rng, n, shards):
            lists = [oracle.dcp_local_topk(scores, n, blocks)[0] for blocks in split]
            assert list(oracle.dcp_merge(scores, n, lists)) == list(want)


def test_dcp_local_lists_by_hand():
    # n = 20 eligible blocks, forced block 19; shard A holds 0..9, shard B 10..24 (its blocks
    # 20..24 are past the token and never eligible)
    scores = np.zeros(25)
    scores[[3, 7, 12, 19]] = [5.0, 5.0, 9.0, -100.0]
    scores[20:] = 50.0
    ids_a, forced_a = oracle.dcp_local_topk(scores, 20, range(0, 10), topk=3)
    assert ids_a == [0, 3, 7] and forced_a == [False] * 3  # 5, 5, then the lowest of the zeros
    ids_b, forced_b = oracle.dcp_local_topk(scores, 20, range(10, 25), topk=3)
    assert ids_b == [10, 12, 19] and forced_b == [False, False, True]  # forced first despite -100
    # merge: forced 19, then 12 (9.0), then the tie of 3 and 7 at 5.0 goes to the lower id
    assert list(oracle.dcp_merge(scores, 20, [ids_a, ids_b], topk=3)) == [3, 12, 19]
    assert list(oracle.dcp_merge(scores, 20, [[], [19]], topk=3)) == [19, -1, -1]


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


def test_index_scores_lse_closed_forms():
    # "MiniMax M3 on vLLM", section "Prefill execution": the block reduction may be log-sum-exp.
    # Keys that quantize exactly make every token score exact: block 0 holds 128 equal scores
    # (LSE = s + log 128), block 1 a single valid token (LSE = its score), block 2 nothing
    # valid (-inf); and the max is never above the LSE nor the LSE above max + log(count).
    T = 129
    w = np.array([1.0, -0.5, 6.0, 0.0] * 32, np.float32)
    ik = np.tile(w, (T, 1))
    codes, scales = oracle.quantize(ik)
    assert np.array_equal(oracle.dequantize(codes, scales), ik.astype(np.float64))
    qv = np.tile(np.array([0.5, 1.0, 0.25, 3.0], np.float32), 32)
    qb = _bf16_bits(np.tile(qv, (1, 4, 1)))
    lse = oracle.index_scores_lse(qb, codes, scales, T, 1, 3)
    s = float(np.dot(w.astype(np.float64), qv.astype(np.float64)))
    assert np.allclose(lse[0, :, 0], s + math.log(128), rtol=0, atol=1e-12)
    assert np.all(lse[0, :, 1] == s)
    assert np.all(np.isneginf(lse[0, :, 2]))
    rng = np.random.default_rng(3)
    ik = rng.standard_normal((700, 128)).astype(np.float32)
    codes, scales = oracle.quantize(ik)
    qb = _bf16_bits(rng.standard_normal((2, 4, 128)))
    mx = oracle.index_scores(qb, codes, scales, 700, 2, 6)
    lse = oracle.index_scores_lse(qb, codes, scales, 700, 2, 6)
    fin = np.isfinite(mx)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(lse[fin] >= mx[fin]) and np.all(lse[fin] <= mx[fin] + math.log(128) + 1e-12)


def test_causal_mask_inside_last_block():
    # q = 4 draft tokens in the last block: token j sees keys up to T - 4 + j only
    T, q = 256, 4
    ik = np.zeros((T, 128), np.float32)
    ik[T - 1] = 1.5                                 # only the very last key is non-zero (exact)
    codes, scales = oracle.quantize(ik)
    qb = _bf16_bits(np.ones((q, 4, 128)))
    got = oracle.index_scores(qb, codes, scales, T, q, 2)
    assert list(got[:, 0, 1]) == [0.0, 0.0, 0.0, 192.0]
