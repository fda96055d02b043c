"""Kernel paths that ordinary seeded inputs never reach, against the oracle (needs an MI355X).

1. Query rows with a dynamic range too wide for fp16. The decode indexer and the attention scale
   each query row by a power of two into fp16 for the matrix cores; a row with values more than
   about 2^30 apart cannot convert exactly, and its wavefront then runs the bf16 matrix-core path
   (same exact products, fp32 sums). Every N(0,1) row converts, so only constructed rows reach
   that path; each test asserts on the host that its rows do not convert exactly by the rule the
   kernels apply (largest magnitude scaled into [2^14, 2^15)).
2. Selection rows of more than 4,097 blocks (contexts past 524,416 tokens, up to the 1M-token
   contexts of "MiniMax M3 on vLLM"): the workgroup radix select, both with the keys held in
   registers (up to 4,096 candidates) and re-read from memory, on constructed tie, signed-zero
   and -inf rows, bit for bit against the oracle. Rows of 1,026 to 4,097 blocks in the fused
   selection + attention call, whose four wavefronts share the selection (a quarter of the row
   each, then a rank among their 60 candidates): ids bit for bit against the oracle and
   msa_block_topk, output bit for bit against msa_sparse_attn_decode on those ids.
3. Pools whose bytes past every context length are 0xFF (E4M3 NaN scales): the attention must
   ignore them (a zero probability times a NaN value would still be NaN), as must the indexer.
"""
import sys

import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from msa_testlib import DeviceWorkload, bf16_to_f64, check_step_against_oracle
from test_gpu_selection import _patterns

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fp16_exact(row: np.ndarray) -> bool:
    """Whether a bf16 row (as fp32 values) converts exactly to fp16 once scaled by the power of
    two that puts its largest magnitude in [2^14, 2^15)."""
    mx = float(np.abs(row).max())
    if mx == 0.0:
        return True
    e = int(np.frexp(np.float32(mx))[1])  # mx in [2^(e-1), 2^e)
    scaled = np.ldexp(row.astype(np.float64), 15 - e).astype(np.float32)
    return bool(np.array_equal(scaled.astype(np.float16).astype(np.float32), scaled))


def _wide_row(rng, n=128) -> torch.Tensor:
    """One value of 1 and the rest N(0,1) * 1e-12: a relative range of about 2^40, in bf16."""
    x = rng.standard_normal(n).astype(np.float32) * np.float32(1e-12)
    x[rng.integers(0, n)] = 1.0
    return torch.from_numpy(x).to(torch.bfloat16)


WIDE_CASES = {
    # (config, overrides, [(token row, group) of q_idx], [(token row, head range) of q])
    "q1_batched": (2, dict(batch=3, ctx=5000), [(1, 2)], [(0, range(16, 32)), (2, range(48, 64))]),
    "q4_spec": (3, dict(batch=2, ctx=6000), [(1, 2), (4, 0)], [(2, range(16, 32)), (7, range(0, 16))]),
    "q16_gemm": (3, dict(batch=1, ctx=6000, q_len=16), [(3, 1), (15, 3)], [(5, range(32, 48))]),
    # 16 sequences: the union attention kernel (wide rows in both halves of the row tiles)
    "q4_union": (3, dict(batch=16, ctx=2000), [(9, 1)], [(1, range(16, 32)), (62, range(48, 64))]),
}


@pytest.mark.parametrize("name", sorted(WIDE_CASES))
def test_wide_range_queries_take_the_bf16_path(name):
    cfg, kw, qi_rows, q_rows = WIDE_CASES[name]
    _log(f"[wide {name}] config {cfg} {kw}")
    w = mi.make_workload(cfg, **kw)
    rng = np.random.default_rng(17)
    for r, g in qi_rows:
        w.q_idx[r, g] = _wide_row(rng)
        assert not _fp16_exact(w.q_idx[r, g].float().numpy()), (name, "q_idx", r, g)
    for r, heads in q_rows:
        for h in heads:
            w.q[r, h] = _wide_row(rng)
        assert not _fp16_exact(w.q[r, heads[0]].float().numpy()), (name, "q", r)
    # an ordinary row of the same workload still converts (the fp16 path runs beside it)
    assert _fp16_exact(w.q[0, 0].float().numpy())
    g = DeviceWorkload(w)
    out = g.run()
    exempt = check_step_against_oracle(w, g.step.block_scores.cpu().numpy(),
                                       g.step.block_ids.cpu().numpy(), bf16_to_f64(out),
                                       max_tokens=16)
    _log(f"[wide {name}] ok, {exempt} rows below margin")


@pytest.mark.parametrize("max_blocks", [4098, 8192])
def test_radix_selection_of_long_rows(max_blocks):
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(3 + max_blocks)
    pats = _patterns(max_blocks, rng)
    # eligible counts on both sides of 4,097 (the wavefront kernel's limit) and of 4,096
    # candidates (keys in registers vs re-read from memory)
    n_list = [16, 17, 1000, 4096, 4097, 4098, 4099, max_blocks - 1, max_blocks]
    n_list = sorted(set(n for n in n_list if n <= max_blocks))
    rows = [pats[(i * 4 + g) % len(pats)] for i in range(len(n_list)) for g in range(4)]
    scores = np.stack(rows).reshape(len(n_list), 4, max_blocks).astype(np.float32)
    ctx = torch.tensor([128 * (n - 1) + 1 for n in n_list], dtype=torch.int32, device="cuda")
    table = torch.zeros((len(n_list), max_blocks), dtype=torch.int32, device="cuda")
    b = msa.Batch(table, ctx, 1)
    s_dev = torch.from_numpy(scores).cuda()
    ids = torch.full((len(n_list), 4, 16), -7, dtype=torch.int32, device="cuda")
    _log(f"[radix {max_blocks}] msa_block_topk")
    msa.msa_block_topk(s_dev, b, 16, ids)
    # the fused call, which runs the same selection kernel for rows this long, then the
    # attention over an all-zero one-page cache (only its ids output is checked here)
    cache = msa.Cache.allocate(1)
    q = torch.zeros((len(n_list), 64, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    ws_bytes = msa.msa_sparse_attn_workspace_bytes(b)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    ids2 = torch.full_like(ids, -7)
    _log(f"[radix {max_blocks}] msa_select_attn_decode")
    msa.msa_select_attn_decode(cache, b, s_dev, 16, ids2, q, 0.088, out, ws)
    torch.cuda.synchronize()
    for path, t in (("topk", ids), ("select_attention", ids2)):
        got = t.cpu().numpy()
        for i, n in enumerate(n_list):
            for g in range(4):
                want, _ = oracle.block_topk(scores[i, g].astype(np.float64), n)
                assert np.array_equal(got[i, g], want), (path, max_blocks, n, g, got[i, g], want)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("max_blocks", [1026, 2500, 4097])
def test_fused_selection_of_rows_up_to_4097_blocks(max_blocks):
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(11 + max_blocks)
    pats = _patterns(max_blocks, rng)
    # eligible counts on both sides of 1,025 (one wavefront's selection) and of each quarter
    n_list = [16, 17, 1024, 1025, 1026, 1100, 2048, 2049, 4096, 4097]
    n_list = sorted(set(n for n in n_list if n <= max_blocks))
    assert len(n_list) * 4 < 512  # four splits: the path under test
    rows = [pats[(i * 4 + g) % len(pats)] for i in range(len(n_list)) for g in range(4)]
    scores = np.stack(rows).reshape(len(n_list), 4, max_blocks).astype(np.float32)
    ctx = torch.tensor([128 * (n - 1) + 1 for n in n_list], dtype=torch.int32, device="cuda")
    # four pages of seeded NVFP4 data, block i of every sequence on page i % 4
    pages = 4
    cache = msa.Cache.allocate(pages)
    g = torch.Generator().manual_seed(5 + max_blocks)
    slots = torch.arange(pages * 128, dtype=torch.int64, device="cuda")
    kv = lambda: torch.randn((pages * 128, 4, 128), generator=g).cuda()
    msa.msa_kv_insert_nvfp4(cache, slots, kv(), kv(), torch.randn((pages * 128, 128), generator=g).cuda())
    table = (torch.arange(max_blocks, dtype=torch.int32, device="cuda") % pages).repeat(len(n_list), 1)
    b = msa.Batch(table.contiguous(), ctx, 1)
    s_dev = torch.from_numpy(scores).cuda()
    q = torch.randn((len(n_list), 64, 128), generator=g).to(torch.bfloat16).cuda()
    ids = torch.full((len(n_list), 4, 16), -7, dtype=torch.int32, device="cuda")
    ids2 = torch.full_like(ids, -7)
    out = torch.empty_like(q)
    out2 = torch.empty_like(q)
    ws_bytes = msa.msa_sparse_attn_workspace_bytes(b)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    _log(f"[fused long {max_blocks}] msa_block_topk + msa_sparse_attn_decode")
    msa.msa_block_topk(s_dev, b, 16, ids)
    msa.msa_sparse_attn_decode(cache, b, q, ids, 0.088, out, ws)
    _log(f"[fused long {max_blocks}] msa_select_attn_decode")
    msa.msa_select_attn_decode(cache, b, s_dev, 16, ids2, q, 0.088, out2, ws)
    torch.cuda.synchronize()
    got, got2 = ids.cpu().numpy(), ids2.cpu().numpy()
    for i, n in enumerate(n_list):
        for gr in range(4):
            want, _ = oracle.block_topk(scores[i, gr].astype(np.float64), n)
            assert np.array_equal(got[i, gr], want), ("topk", max_blocks, n, gr)
            assert np.array_equal(got2[i, gr], want), ("fused", max_blocks, n, gr, got2[i, gr], want)
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


FILL_CASES = {
    # partial last blocks everywhere; decode (q = 1, 4) and the token-tile attention (q = 256,
    # 1,024 rows), fused step and the four separate calls
    "ragged_q1": (4, dict(ctx_lens=[3000, 129, 7777, 1, 17 * 128 + 5, 2048 + 77])),
    "spec_q4": (3, dict(batch=2, ctx_lens=[6000, 2 * 128 + 2])),
    "prefill_q256": (5, dict(batch=1, ctx=2048 + 256 + 50, q_len=256)),
    "union_q4": (3, dict(batch=16, ctx_lens=[300 + 97 * i for i in range(16)])),
}


@pytest.mark.parametrize("mode", ["step", "separate"])
@pytest.mark.parametrize("name", sorted(FILL_CASES))
def test_unwritten_bytes_past_the_context_are_ignored(name, mode):
    cfg, kw = FILL_CASES[name]
    _log(f"[fill {name} {mode}] config {cfg} {kw}")
    w = mi.make_workload(cfg, **kw)
    g = DeviceWorkload(w, mode=mode, fill=0xFF)
    # the last page of some sequence does hold 0xFF bytes past its context
    b = int(np.argmax([(t % 128) != 0 for t in w.ctx_lens]))
    page = int(w.block_table[b, (w.ctx_lens[b] - 1) // 128])
    assert int(g.cache.v[page, 0, -1]) == 0xFF and int(g.cache.k[page, 0, -1]) == 0xFF
    out = g.run()
    assert torch.isfinite(out.float()).all(), (name, mode, "non-finite outputs")
    scores = g.step.block_scores.cpu().numpy()
    assert not np.isnan(scores).any(), (name, mode, "NaN scores")
    check_step_against_oracle(w, scores, g.step.block_ids.cpu().numpy(), bf16_to_f64(out))
    _log(f"[fill {name} {mode}] ok")


@pytest.mark.parametrize("batch,q_len", [(2, 4), (16, 4)], ids=["per_token_splits", "union"])
def test_workspace_recovers_after_counters_were_left_set(batch, q_len):
    """A workspace whose split counters were left non-zero (as an interrupted call would leave
    them) gives unspecified outputs but no fault; zero-filling it again, as the header says,
    restores the exact results (per-token kernel with four splits, and the union kernel)."""
    import block_sparse_attention_nvfp4_amd as msa
    _log(f"workspace recovery batch={batch} q={q_len}")
    w = mi.make_workload(3, batch=batch, ctx=2600, q_len=q_len, seed=91)
    d = DeviceWorkload(w)
    msa.msa_kv_insert_nvfp4(d.cache, d.new_slots, d.new_k, d.new_v, d.new_ik)
    rows = batch * q_len
    scores = torch.empty((rows, 4, w.max_blocks), dtype=torch.float32, device="cuda")
    msa.msa_indexer_score(d.cache, d.batch, d.q_idx, scores)
    ids = torch.empty((rows, 4, 16), dtype=torch.int32, device="cuda")
    msa.msa_block_topk(scores, d.batch, 16, ids)
    need = msa.msa_sparse_attn_workspace_bytes(d.batch)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    scale = msa.default_softmax_scale()
    ref = torch.empty((rows, 64, 128), dtype=torch.bfloat16, device="cuda")
    msa.msa_sparse_attn_decode(d.cache, d.batch, d.q, ids, scale, ref, ws)
    again = torch.empty_like(ref)
    msa.msa_sparse_attn_decode(d.cache, d.batch, d.q, ids, scale, again, ws)  # left zeroed
    ws.fill_(1)  # every counter (and partial) byte set: 0x01010101 per counter
    junk = torch.zeros_like(ref)
    msa.msa_sparse_attn_decode(d.cache, d.batch, d.q, ids, scale, junk, ws)
    torch.cuda.synchronize()
    ws.zero_()
    fixed = torch.empty_like(ref)
    msa.msa_sparse_attn_decode(d.cache, d.batch, d.q, ids, scale, fixed, ws)
    torch.cuda.synchronize()
    r = ref.view(torch.int16).cpu().numpy()
    assert np.array_equal(again.view(torch.int16).cpu().numpy(), r)
    assert np.array_equal(fixed.view(torch.int16).cpu().numpy(), r)


@pytest.mark.parametrize("init_blocks,local_blocks", [(2, 2), (0, 3), (4, 1)])
def test_window_selection_drives_the_attention(init_blocks, local_blocks):
    """The selection knobs end to end at 16 blocks per row: msa_block_topk_window's ids (bit for
    bit those of oracle.block_topk_variant on the same scores) feed msa_sparse_attn_decode, whose
    outputs match the oracle's attention over those ids."""
    import block_sparse_attention_nvfp4_amd as msa
    from msa_testlib import check_attention, oracle_sequence
    _log(f"window selection init={init_blocks} local={local_blocks}")
    w = mi.make_workload(3, batch=3, ctx_lens=[5000, 128 * 23 + 7, 2100], q_len=4, seed=17)
    d = DeviceWorkload(w)
    msa.msa_kv_insert_nvfp4(d.cache, d.new_slots, d.new_k, d.new_v, d.new_ik)
    rows = w.batch * w.q_len
    scores = torch.empty((rows, 4, w.max_blocks), dtype=torch.float32, device="cuda")
    msa.msa_indexer_score(d.cache, d.batch, d.q_idx, scores)
    ids = torch.full((rows, 4, 16), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_topk_window(scores, d.batch, 16, init_blocks, local_blocks, ids)
    ws_bytes = msa.msa_sparse_attn_workspace_bytes(d.batch)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((rows, 64, 128), dtype=torch.bfloat16, device="cuda")
    msa.msa_sparse_attn_decode(d.cache, d.batch, d.q, ids, msa.default_softmax_scale(), out,
                               ws if ws_bytes else None)
    torch.cuda.synchronize()
    s_h, ids_h = scores.cpu().numpy(), ids.cpu().numpy()
    got = bf16_to_f64(out)
    for b in range(w.batch):
        T = w.ctx_lens[b]
        for j in range(w.q_len):
            r = b * w.q_len + j
            n = (T - w.q_len + j) // 128 + 1
            for g in range(4):
                want = oracle.block_topk_variant(s_h[r, g], n, 16, init_blocks, local_blocks)
                assert list(ids_h[r, g]) == list(want), (r, g)
        rr = slice(b * w.q_len, (b + 1) * w.q_len)
        ref = oracle_sequence(w, b, attention_tokens=list(range(w.q_len)), ids_override=ids_h[rr])
        check_attention(got[rr], ref["attention"])
