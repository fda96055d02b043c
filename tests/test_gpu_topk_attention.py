"""Attention over selections of 1 to 64 blocks per row, against the oracle (needs an MI355X).

"MiniMax M3 on vLLM", section "MSA mechanism", makes the number of kept blocks and the init and
local windows configuration knobs; "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA
primer", fixes what follows the selection: exact attention over the kept blocks. Here
msa_block_topk_window's ids (bit for bit those of oracle.block_topk_variant on the same scores)
drive msa_sparse_attn_decode_topk end to end, and its outputs are checked against the oracle's
attention over those ids. The batch shapes take each split count of the per-token kernel
(4 splits below 512 rows, 2 below 1,024, then 1), so a wavefront streams from 1 up to 16
blocks in turn, and each split count of the union kernel, which rows of up to 16 ids take where
the 16-id call takes it (2 to 4 query tokens per sequence, 16 sequences and more: 4 splits per
(sequence, group) at 16 sequences, 2 at 32, one from 64 on). With 16 ids per row the call must
give msa_sparse_attn_decode's bits wherever both run the same kernel. Rows that list a block twice,
or hold -1 or an id past the block table, must be attended as the formula says (a repeated
block's keys count twice, the others are skipped) on both kernels. At the benchmark's window
workload (8 x 131,072 tokens, 4 query tokens, top-64 with 1 init and 2 local blocks) the ids are
checked on every row and the attention on sampled sequences.
"""
import sys

import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from msa_testlib import DeviceWorkload, bf16_to_f64, check_attention, oracle_sequence

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# name: (config, workload overrides, topk, init_blocks, local_blocks, sequences checked
# against the oracle (None: all))
CASES = {
    "k1_q4": (3, dict(batch=3, ctx_lens=[5000, 128 * 23 + 7, 2100], q_len=4, seed=17), 1, 0, 1, None),
    "k8_q4": (3, dict(batch=3, ctx_lens=[5000, 128 * 23 + 7, 2100], q_len=4, seed=17), 8, 1, 1, None),
    "k32_q4": (3, dict(batch=3, ctx_lens=[9000, 128 * 40 + 1, 2100], q_len=4, seed=19), 32, 2, 2, None),
    "k64_q4": (3, dict(batch=2, ctx_lens=[10000, 128 * 70 + 5], q_len=4, seed=23), 64, 4, 1, None),
    "k64_q1": (2, dict(batch=3, ctx_lens=[12000, 128 * 64, 700], q_len=1, seed=29), 64, 0, 1, None),
    "k40_q3": (3, dict(batch=2, ctx_lens=[7000, 6000], q_len=3, seed=31), 40, 3, 2, None),
    # 520 rows: two splits, 6 slots per wavefront
    "k48_q5_2split": (3, dict(batch=26, ctx_lens=[9000, 8000] + [1100] * 24, q_len=5, seed=37),
                      48, 2, 3, [0, 1, 25]),
    # 1,040 rows: one split, 16 slots per wavefront
    "k64_q5_1split": (3, dict(batch=52, ctx_lens=[9500, 8800] + [1000] * 50, q_len=5, seed=41),
                      64, 0, 1, [0, 1, 51]),
    # 2 query tokens, 4 splits of the per-token kernel
    "k24_q2": (3, dict(batch=4, ctx_lens=[6000, 128 * 30 + 3, 2100, 300], q_len=2, seed=43),
               24, 1, 2, None),
    # 32 sequences of 4 query tokens with 64 ids: the per-token kernel
    "k64_q4_b32": (3, dict(batch=32, ctx_lens=[9000, 8500] + [1300] * 30, q_len=4, seed=53),
                   64, 2, 2, [0, 1, 31]),
    # 16 sequences: the union kernel with 8 ids per row, 4 splits
    "k8_q3_union16": (3, dict(batch=16, ctx_lens=[5000, 4000] + [1500] * 14, q_len=3, seed=47),
                      8, 1, 1, [0, 1, 15]),
    # 32 sequences: the union kernel with 12 ids per row, 2 splits
    "k12_q4_union32": (3, dict(batch=32, ctx_lens=[9000, 8500] + [1300] * 30, q_len=4, seed=53),
                       12, 2, 2, [0, 1, 31]),
    # 64 sequences: the union kernel with 5 ids per row, one split
    "k5_q2_union64": (3, dict(batch=64, ctx_lens=[9000] + [700] * 63, q_len=2, seed=59),
                      5, 1, 1, [0, 63]),
}


def _setup(cfg, kw):
    import block_sparse_attention_nvfp4_amd as msa
    w = mi.make_workload(cfg, **kw)
    d = DeviceWorkload(w)
    msa.msa_kv_insert_nvfp4(d.cache, d.new_slots, d.new_k, d.new_v, d.new_ik)
    rows = w.batch * w.q_len
    scores = torch.empty((rows, 4, w.max_blocks), dtype=torch.float32, device="cuda")
    msa.msa_indexer_score(d.cache, d.batch, d.q_idx, scores)
    ws_bytes = msa.msa_sparse_attn_workspace_bytes(d.batch)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
    return w, d, scores, ws


@pytest.mark.parametrize("name", list(CASES))
def test_any_topk_selection_drives_the_attention(name):
    import block_sparse_attention_nvfp4_amd as msa
    cfg, kw, topk, init, local, check = CASES[name]
    _log(f"topk attention case {name}: topk={topk} init={init} local={local}")
    w, d, scores, ws = _setup(cfg, kw)
    rows = w.batch * w.q_len
    ids = torch.full((rows, 4, topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk_window(scores, d.batch, topk, init, local, ids)
    out = torch.full((rows, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    msa.msa_sparse_attn_decode_topk(d.cache, d.batch, d.q, ids, msa.default_softmax_scale(), out, ws)
    torch.cuda.synchronize()
    s_h, ids_h = scores.cpu().numpy(), ids.cpu().numpy()
    got = bf16_to_f64(out)
    assert np.isfinite(got).all()
    for b in range(w.batch):
        T = w.ctx_lens[b]
        for j in range(w.q_len):
            r = b * w.q_len + j
            n = (T - w.q_len + j) // 128 + 1
            for g in range(4):
                want = oracle.block_topk_variant(s_h[r, g], n, topk, init, local)
                assert list(ids_h[r, g]) == list(want), (r, g)
    kept = (ids_h >= 0).sum(axis=2)
    assert kept.max() == min(topk, max((t - 1) // 128 + 1 for t in w.ctx_lens))
    for b in (range(w.batch) if check is None else check):
        rr = slice(b * w.q_len, (b + 1) * w.q_len)
        ref = oracle_sequence(w, b, attention_tokens=list(range(w.q_len)), ids_override=ids_h[rr])
        check_attention(got[rr], ref["attention"])


@pytest.mark.parametrize("name", ["k8_q4", "k48_q5_2split", "k64_q5_1split", "k8_q3_union16"])
def test_sixteen_ids_match_the_fixed_size_call(name):
    """topk = 16 through the sized call gives msa_sparse_attn_decode's bits (both run the
    per-token kernel under 16 sequences or at 5 query tokens per sequence, and the union kernel
    at 16 sequences of 3 query tokens)."""
    import block_sparse_attention_nvfp4_amd as msa
    cfg, kw, _, _, _, _ = CASES[name]
    _log(f"topk attention 16 ids vs fixed call: {name}")
    w, d, scores, ws = _setup(cfg, kw)
    rows = w.batch * w.q_len
    ids = torch.empty((rows, 4, 16), dtype=torch.int32, device="cuda")
    msa.msa_block_topk(scores, d.batch, 16, ids)
    scale = msa.default_softmax_scale()
    a = torch.empty((rows, 64, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    msa.msa_sparse_attn_decode(d.cache, d.batch, d.q, ids, scale, a, ws)
    msa.msa_sparse_attn_decode_topk(d.cache, d.batch, d.q, ids, scale, b, ws)
    torch.cuda.synchronize()
    assert np.array_equal(a.view(torch.int16).cpu().numpy(), b.view(torch.int16).cpu().numpy())



# name: (config, workload overrides, topk); the per-token kernel runs the first two, the union
# kernel the others
EDIT_CASES = {
    "per_token_q5": (3, dict(batch=3, ctx_lens=[5000, 128 * 23 + 7, 2100], q_len=5, seed=61), 20),
    "per_token_q4": (3, dict(batch=3, ctx_lens=[5000, 128 * 23 + 7, 2100], q_len=4, seed=61), 16),
    "union16_q3": (3, dict(batch=16, ctx_lens=[4000, 3000] + [1200] * 14, q_len=3, seed=67), 16),
    "union32_q4_k10": (3, dict(batch=32, ctx_lens=[4000, 3000] + [1200] * 30, q_len=4, seed=71), 10),
}


@pytest.mark.parametrize("name", list(EDIT_CASES))
def test_repeated_and_skipped_ids(name):
    """Window ids edited on the host: in every row entry 1 repeats entry 0, entry 2 is past the
    block table, entry 3 is -1 (the rest as selected). The oracle attends each listed block
    once per listing and skips the others; both kernels must agree with it."""
    import block_sparse_attention_nvfp4_amd as msa
    cfg, kw, topk = EDIT_CASES[name]
    _log(f"topk attention with edited ids: {name}")
    w, d, scores, ws = _setup(cfg, kw)
    rows = w.batch * w.q_len
    ids = torch.full((rows, 4, topk), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk_window(scores, d.batch, topk, 1, 1, ids)
    ids_h = ids.cpu().numpy()
    ids_h[:, :, 1] = ids_h[:, :, 0]
    ids_h[:, :, 2] = w.max_blocks + 3
    ids_h[:, :, 3] = -1
    ids = torch.from_numpy(ids_h).cuda()
    out = torch.full((rows, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    msa.msa_sparse_attn_decode_topk(d.cache, d.batch, d.q, ids, msa.default_softmax_scale(), out, ws)
    torch.cuda.synchronize()
    got = bf16_to_f64(out)
    assert np.isfinite(got).all()
    seqs = range(w.batch) if w.batch <= 4 else [0, 1, w.batch - 1]
    for b in seqs:
        rr = slice(b * w.q_len, (b + 1) * w.q_len)
        ref = oracle_sequence(w, b, attention_tokens=list(range(w.q_len)), ids_override=ids_h[rr])
        check_attention(got[rr], ref["attention"])


def test_window64_at_full_size():
    """The benchmark's window workload at full size: 8 sequences of 131,072 tokens, 4 query
    tokens each, top-64 with the first block and the last 2 kept. The ids match the oracle's
    selection on the device's scores on every row (the same scores, so bit for bit), and the
    attention matches the oracle's over those ids on the first and last sequences."""
    import block_sparse_attention_nvfp4_amd as msa
    _log("topk attention: window top-64 at full size (8 x 131,072 tokens, 4 query tokens)")
    w = mi.full_workload(3)
    d = DeviceWorkload(w)
    msa.msa_kv_insert_nvfp4(d.cache, d.new_slots, d.new_k, d.new_v, d.new_ik)
    rows = w.batch * w.q_len
    scores = torch.empty((rows, 4, w.max_blocks), dtype=torch.float32, device="cuda")
    msa.msa_indexer_score(d.cache, d.batch, d.q_idx, scores)
    ws_bytes = msa.msa_sparse_attn_workspace_bytes(d.batch)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    ids = torch.full((rows, 4, 64), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk_window(scores, d.batch, 64, 1, 2, ids)
    out = torch.full((rows, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    msa.msa_sparse_attn_decode_topk(d.cache, d.batch, d.q, ids, msa.default_softmax_scale(), out, ws)
    torch.cuda.synchronize()
    s_h, ids_h = scores.cpu().numpy(), ids.cpu().numpy()
    got = bf16_to_f64(out)
    assert np.isfinite(got).all()
    for b in range(w.batch):
        T = w.ctx_lens[b]
        for j in range(w.q_len):
            r = b * w.q_len + j
            n = (T - w.q_len + j) // 128 + 1
            for g in range(4):
                want = oracle.block_topk_variant(s_h[r, g], n, 64, 1, 2)
                assert list(ids_h[r, g]) == list(want), (r, g)
    for b in (0, w.batch - 1):
        rr = slice(b * w.q_len, (b + 1) * w.q_len)
        ref = oracle_sequence(w, b, attention_tokens=list(range(w.q_len)), ids_override=ids_h[rr])
        d_max, _ = check_attention(got[rr], ref["attention"])
        _log(f"  sequence {b}: attention worst |d| {d_max:.3e}")


@pytest.mark.parametrize("name", ["k64_q4", "k40_q3", "k8_q3_union16"])
def test_window_step_matches_the_three_calls(name):
    """msa_decode_step_window gives, bit for bit, the block scores, ids, outputs and cache bytes
    of msa_insert_indexer_score, msa_block_topk_window and msa_sparse_attn_decode_topk called
    one after the other on the same inputs."""
    import block_sparse_attention_nvfp4_amd as msa
    cfg, kw, topk, init, local, _ = CASES[name]
    _log(f"window step vs the three calls: {name}")
    w = mi.make_workload(cfg, **kw)
    g = DeviceWorkload(w, snapshot=True)
    rows = w.batch * w.q_len
    ws_bytes = msa.msa_sparse_attn_workspace_bytes(g.batch)
    scale = msa.default_softmax_scale()
    res = []
    for fused in (False, True):
        g.restore_prefix()
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        scores = torch.full((rows, 4, w.max_blocks), float("nan"), dtype=torch.float32, device="cuda")
        ids = torch.full((rows, 4, topk), -7, dtype=torch.int32, device="cuda")
        out = torch.full((rows, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        if fused:
            msa.msa_decode_step_window(g.cache, g.batch, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q,
                                       topk, init, local, scale, scores, ids, out, ws)
        else:
            msa.msa_insert_indexer_score(g.cache, g.batch, g.new_k, g.new_v, g.new_ik, g.q_idx,
                                         scores)
            msa.msa_block_topk_window(scores, g.batch, topk, init, local, ids)
            msa.msa_sparse_attn_decode_topk(g.cache, g.batch, g.q, ids, scale, out, ws)
        torch.cuda.synchronize()
        res.append([t.clone() for t in (scores, ids, out, g.cache.k, g.cache.v, g.cache.ik)])
    assert torch.isfinite(res[1][2].float()).all()
    for i, (a, b) in enumerate(zip(*res)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (name, i)
