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
