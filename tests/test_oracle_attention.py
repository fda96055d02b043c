"""Pins of the oracle's sparse GQA attention.

Sources: "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer" and its Figure 1
(each query head of a GQA group attends exactly to its group's selected blocks; with at most
16 blocks of context every block is selected, so sparse equals dense); "MiniMax M3 on vLLM",
section "Prefill execution" (the sparse result equals dense attention restricted to the
selected set). Closed forms: constant V gives that constant; Q = 0 gives the mean of V over
the attended keys; one attended key gives its V.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_kv(T, seed, const_v=None):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, 4, 128)).astype(np.float32)
    v = rng.standard_normal((T, 4, 128)).astype(np.float32) if const_v is None else \
        np.full((T, 4, 128), const_v, np.float32)
    kc, ks = oracle.quantize(k)
    vc, vs = oracle.quantize(v)
    return kc, ks, vc, vs


def numpy_attention(qb, kc, ks, vc, vs, keys_per_group, scale):
    """Independent restatement: softmax over an explicit key list per group, numpy ops."""
    K = oracle.dequantize(kc, ks)   # [T][4][128]
    V = oracle.dequantize(vc, vs)
    Q = bits_to_f64(qb)
    out = np.zeros((64, 128))
    for h in range(64):
        g = h // 16
        t = np.asarray(keys_per_group[g], np.int64)
        if len(t) == 0:
            continue
        lg = K[t, g] @ Q[h] * scale
        w = np.exp(lg - lg.max())
        out[h] = (w / w.sum()) @ V[t, g]
    return out


@pytest.mark.parametrize("T", [1, 100, 128, 129, 2048, 2047])
def test_sparse_equals_dense_when_at_most_16_blocks(T):
    kc, ks, vc, vs = make_kv(T, T)
    qb = bits(np.random.default_rng(T + 1).standard_normal((64, 128)))
    p = T - 1
    n = p // 128 + 1
    assert n <= 16
    scores = np.random.default_rng(5).standard_normal(n)
    ids, _ = oracle.block_topk(scores, n)
    sel = np.tile(ids, (4, 1))
    s = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, sel, p, oracle.default_scale())
    d = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, oracle.dense_ids(p), p, oracle.default_scale())
    assert np.array_equal(s, d)
    ref = numpy_attention(qb, kc, ks, vc, vs, [list(range(T))] * 4, oracle.default_scale())
    assert np.allclose(s, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_sparse_equals_dense_restricted_to_selection(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(2200, 5000))
    q_len = int(rng.integers(1, 5))
    j = int(rng.integers(0, q_len))
    p = T - q_len + j
    n = p // 128 + 1
    kc, ks, vc, vs = make_kv(T, seed + 100)
    qb = bits(rng.standard_normal((64, 128)))
    sel = np.stack([oracle.block_topk(rng.standard_normal(n), n)[0] for _ in range(4)])
    got = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, sel, p, 0.0883883)
    keys = [[t for b in sel[g] if b >= 0 for t in range(b * 128, min(b * 128 + 128, p + 1))] for g in range(4)]
    assert all(len(k) <= 2048 for k in keys)
    ref = numpy_attention(qb, kc, ks, vc, vs, keys, 0.0883883)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_constant_v_gives_constant_output():
    T = 3000
    kc, ks, vc, vs = make_kv(T, 1, const_v=1.5)
    qb = bits(np.random.default_rng(2).standard_normal((64, 128)) * 4)
    n = (T - 1) // 128 + 1
    sel = np.tile(oracle.block_topk(np.arange(n, dtype=np.float64), n)[0], (4, 1))
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, sel, T - 1, oracle.default_scale())
    assert np.allclose(out, 1.5, rtol=0, atol=1e-13)


def test_zero_query_gives_mean_of_selected_values():
    T = 1500
    kc, ks, vc, vs = make_kv(T, 3)
    qb = bits(np.zeros((64, 128)))
    sel = np.array([[0, 5, 11, -1] + [-1] * 12] * 4, np.int32)
    p = T - 1                          # block 11 holds tokens 1408..1499: partial
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, sel, p, oracle.default_scale())
    V = oracle.dequantize(vc, vs)
    toks = list(range(0, 128)) + list(range(640, 768)) + list(range(1408, 1500))
    for g in range(4):
        assert np.allclose(out[16 * g:16 * g + 16], V[toks, g].mean(0), rtol=1e-12, atol=1e-13)


def test_single_valid_key_returns_its_value():
    T = 1
    kc, ks, vc, vs = make_kv(T, 4)
    qb = bits(np.random.default_rng(9).standard_normal((64, 128)))
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, oracle.dense_ids(0), 0, 1.0)
    V = oracle.dequantize(vc, vs)
    for h in range(64):
        assert np.array_equal(out[h], V[0, h // 16])


def test_head_to_group_map_is_contiguous():
    # group g's values are vals[g] (each exact in NVFP4): head h must read group h // 16
    T = 200
    vals = [1.5, 3.0, 6.0, 0.75]
    rng = np.random.default_rng(5)
    k = rng.standard_normal((T, 4, 128)).astype(np.float32)
    v = np.stack([np.full((T, 128), vals[g], np.float32) for g in range(4)], axis=1)
    kc, ks = oracle.quantize(k)
    vc, vs = oracle.quantize(v)
    qb = bits(rng.standard_normal((64, 128)))
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, oracle.dense_ids(T - 1), T - 1, 0.1)
    for h in range(64):
        assert np.allclose(out[h], vals[h // 16], atol=1e-13)


# ---------------------------------------------------------------- exact softmax weightings
# The pins below build the NVFP4 caches byte by byte (E4M3 scale byte 0x38 = 1.0 and E2M1
# codes of exact grid values, not through the oracle's quantizer) and bf16 queries whose dot
# products with every key are exact, so the softmax weights follow in closed form from the
# logit differences: a difference of ln r between two keys gives weights in the ratio r.
# One-hot values then expose each key's weight directly in one output dimension. They fail
# for a wrong logit scale (e.g. a doubled scale), a base-2 exponential in place of the natural
# one, a missing max subtraction (logits above 709), a key past the query position or a
# missing key in the denominator.

E2M1_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
SCALE_ONE = 0x38  # E4M3: exponent field 7, mantissa 0 -> 2^0


def hand_cache(T, entries):
    """NVFP4 codes/scales [T][4][64] / [T][4][8], every group of every head scaled by 1.0.

    entries: {(token, dim): value} set in all four KV heads; value on the E2M1 grid.
    """
    codes = np.zeros((T, 4, 64), np.uint8)
    scales = np.full((T, 4, 8), SCALE_ONE, np.uint8)
    for (t, d), x in entries.items():
        nib = E2M1_CODE[abs(x)] | (8 if x < 0 else 0)
        codes[t, :, d // 2] |= nib << (4 * (d % 2))
    return codes, scales


def query_bits(rows):
    """bf16 bit patterns [64][128] of a query whose head h has the (dim -> value) map rows(h);
    every value is a power of two or zero, so it is exact in bf16."""
    q = np.zeros((64, 128), np.float32)
    for h in range(64):
        for d, x in rows(h).items():
            q[h, d] = x
    b = (q.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), q)
    return b


def test_ln3_logit_gap_gives_three_to_one_weights():
    # token 0: key 4 e0, value 6 e0; token 1: key 6 e0, value 6 e1. Query +-e0 per head parity:
    # dot products +-4 and +-6, a gap of 2; scale ln(3)/2 makes the gap ln 3, weights 1/4, 3/4
    # (swapped for the heads with the negated query).
    kc, ks = hand_cache(2, {(0, 0): 4.0, (1, 0): 6.0})
    vc, vs = hand_cache(2, {(0, 0): 6.0, (1, 1): 6.0})
    qb = query_bits(lambda h: {0: 1.0 if h % 2 == 0 else -1.0})
    ids = oracle.dense_ids(1)
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, 2, ids, 1, math.log(3.0) / 2)
    for h in range(64):
        want = np.zeros(128)
        want[0], want[1] = (1.5, 4.5) if h % 2 == 0 else (4.5, 1.5)
        assert np.allclose(out[h], want, rtol=0, atol=1e-12), h
    # the negated scale swaps the weights of every head; scale 0 gives the plain mean
    neg = oracle.sparse_attention_token(qb, kc, ks, vc, vs, 2, ids, 1, -math.log(3.0) / 2)
    zero = oracle.sparse_attention_token(qb, kc, ks, vc, vs, 2, ids, 1, 0.0)
    for h in range(64):
        a, b = (4.5, 1.5) if h % 2 == 0 else (1.5, 4.5)
        assert abs(neg[h, 0] - a) <= 1e-12 and abs(neg[h, 1] - b) <= 1e-12, h
        assert abs(zero[h, 0] - 3.0) <= 1e-12 and abs(zero[h, 1] - 3.0) <= 1e-12, h
        assert np.all(neg[h, 2:] == 0) and np.all(zero[h, 2:] == 0)


def test_geometric_logits_give_one_two_four_sevenths():
    # keys 2, 4, 6 along e0 with query e0: logits 2c, 4c, 6c; c = ln(2)/2 makes consecutive
    # gaps ln 2, so the weights are 1/7, 2/7, 4/7; values 6 e0, 6 e1, 6 e2 show each weight.
    kc, ks = hand_cache(3, {(0, 0): 2.0, (1, 0): 4.0, (2, 0): 6.0})
    vc, vs = hand_cache(3, {(0, 0): 6.0, (1, 1): 6.0, (2, 2): 6.0})
    qb = query_bits(lambda h: {0: 1.0})
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, 3, oracle.dense_ids(2), 2,
                                        math.log(2.0) / 2)
    for h in range(64):
        assert np.allclose(out[h, :3], [6 / 7, 12 / 7, 24 / 7], rtol=0, atol=1e-12), h
        assert np.all(out[h, 3:] == 0)


def test_large_logits_need_the_max_subtraction():
    # query e0 + 2^-10 e1; keys 6 e0 and 6 e0 + 6 e1: dot products 6 and 6 + 6 * 2^-10. With
    # scale ln(3) / (6 * 2^-10) ~ 187.5 the logits are ~1125 and ~1126 (exp overflows fp64
    # without subtracting the maximum) and their gap is ln 3: weights 1/4, 3/4.
    kc, ks = hand_cache(2, {(0, 0): 6.0, (1, 0): 6.0, (1, 1): 6.0})
    vc, vs = hand_cache(2, {(0, 0): 6.0, (1, 1): 6.0})
    qb = query_bits(lambda h: {0: 1.0, 1: 2.0 ** -10})
    scale = math.log(3.0) / (6 * 2.0 ** -10)
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, 2, oracle.dense_ids(1), 1, scale)
    assert np.all(np.isfinite(out))
    for h in range(64):
        assert np.allclose(out[h, :2], [1.5, 4.5], rtol=0, atol=1e-10), h


def test_weights_count_every_visible_key_and_no_later_one():
    # T = 210, query position p = 200 (a draft token: tokens 201..209 exist but come after it).
    # Blocks 0 and 1 selected; every key is 0 except token 5 (6 e0), token 200 (6 e0 + 6 e1) and
    # token 205 (6 e0 + 6 e1 + 6 e2, after the query: must not count). Query e0 + e1, scale
    # ln(127)/6: token 5 has weight 127/Z, token 200 127^2/Z and the other 199 visible keys
    # 1/Z each, Z = 199 + 127 + 127^2.
    T, p = 210, 200
    kc, ks = hand_cache(T, {(5, 0): 6.0, (200, 0): 6.0, (200, 1): 6.0,
                            (205, 0): 6.0, (205, 1): 6.0, (205, 2): 6.0})
    vc, vs = hand_cache(T, {(5, 0): 6.0, (200, 1): 6.0, (205, 2): 6.0})
    qb = query_bits(lambda h: {0: 1.0, 1: 1.0})
    ids = np.array([[0, 1] + [-1] * 14] * 4, np.int32)
    out = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, ids, p, math.log(127.0) / 6)
    Z = 199 + 127 + 127 ** 2
    for h in range(64):
        assert np.allclose(out[h, :3], [6 * 127 / Z, 6 * 127 ** 2 / Z, 0.0], rtol=0, atol=1e-12), h
    # only block 1 selected: token 200 and the 72 zero keys 128..199 remain
    ids1 = np.array([[1] + [-1] * 15] * 4, np.int32)
    out1 = oracle.sparse_attention_token(qb, kc, ks, vc, vs, T, ids1, p, math.log(127.0) / 6)
    Z1 = 72 + 127 ** 2
    for h in range(64):
        assert np.allclose(out1[h, :3], [0.0, 6 * 127 ** 2 / Z1, 0.0], rtol=0, atol=1e-12), h
