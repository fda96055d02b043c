"""HIP path vs the oracle, element by element, on seeded inputs (needs an MI355X).

Quantization and selection are compared bit for bit, index scores within the fp32 accumulation
bound, attention within |d| <= 2e-3 + 1e-2 |ref| per element and 1e-2 relative L2.
Workloads are the five recipes of msa_inputs at reduced sizes that still span several blocks,
a ragged tail, random page permutations and every masking case; the full sizes are covered by
test_gpu_full.py.
"""
import sys

import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from msa_testlib import (DeviceWorkload, bf16_to_f64, check_attention, check_step_against_oracle,
                         gpu_sequence_caches, oracle_sequence, score_tolerance)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, overrides)
    "tiny_full": (1, {}),
    "batched_small": (2, dict(batch=3, ctx=9000)),
    "spec_small": (3, dict(batch=2, ctx=6000)),
    "ragged_small": (4, dict(ctx_lens=[3000, 129, 7777, 1, 17 * 128 + 5, 2048])),
    "prefill_small": (5, dict(batch=1, ctx=2048 + 128, q_len=128)),
    "short_context": (2, dict(batch=2, ctx_lens=[1000, 2048], q_len=1)),
    "spec_at_block_edge": (3, dict(batch=2, ctx_lens=[2 * 128 + 2, 20 * 128 + 3], q_len=4)),
    # 1,024 row groups: one workgroup per row group, no split partials
    "prefill_q256": (5, dict(batch=1, ctx=2048 + 256, q_len=256)),
    # speculative verify with 2, 3, 8 and 16 draft tokens (token tiles of 2 and 4, a partial
    # tile, several tiles), and 17 (the per-token path above 16)
    "spec_q2": (3, dict(batch=2, ctx=5000, q_len=2)),
    "spec_q3": (3, dict(batch=3, ctx_lens=[3000, 4097, 5000], q_len=3)),
    "spec_q8": (3, dict(batch=2, ctx_lens=[4000, 7000], q_len=8)),
    "spec_q16": (3, dict(batch=1, ctx=6000, q_len=16)),
    "spec_q17": (3, dict(batch=1, ctx=6000, q_len=17)),
    # the score-GEMM indexer: a context that is only its query tokens (first token at p = 0),
    # partial last blocks, blocks past the shorter sequences, and 800 rows per sequence (two
    # row ranges, the second partial)
    "prefill_ragged": (5, dict(batch=3, ctx_lens=[40, 700, 3003], q_len=40)),
    # rows of more than 2,048 blocks: a long sequence beside short ones (one of them past every
    # indexer workgroup of its row but the first), the selection of rows past 1,025 blocks
    "long_table": (4, dict(batch=3, ctx_lens=[2100 * 128 + 77, 3000, 129])),
    "prefill_q200": (5, dict(ctx_lens=[2048 + 200, 1500], q_len=200)),
    # 16 or more sequences with 2 to 4 draft tokens: the union kernel (each (sequence, group)
    # reads the union of its drafts' blocks once): 4 and 2 splits per pair, ragged lengths with
    # drafts in two blocks, and one split (64 sequences)
    "union_q4": (3, dict(batch=16, ctx=2600)),
    "union_q2": (3, dict(batch=17, ctx_lens=[2500 + 37 * i for i in range(17)], q_len=2)),
    "union_q3": (3, dict(batch=32, ctx_lens=[258 + 131 * i for i in range(32)], q_len=3)),
    "union_q4_one_split": (3, dict(batch=64, ctx_lens=[130 + 29 * i for i in range(64)])),
    # rows of 1,026 to 4,097 blocks: the selection shared by the attention workgroup's four
    # wavefronts, and indexer workgroups whose blocks all lie past a short sequence's context
    # consecutive drafts whose positions lie in different blocks (127 | 128, 1151 | 1152,
    # 383 | 384), and 6 drafts per sequence
    "spec_pair_straddle": (3, dict(batch=3, ctx_lens=[131, 128 * 9 + 1, 3 * 128 + 3], q_len=4)),
    "spec_q6": (3, dict(batch=2, ctx_lens=[3000, 5100], q_len=6)),
    "ragged_long": (4, dict(batch=3, ctx_lens=[140_001, 2_000, 70_000])),
    "spec_long": (3, dict(batch=2, ctx_lens=[140_000, 131_203], q_len=4)),
}


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=sorted(CASES))
def run(request):
    cfg, kw = CASES[request.param]
    _log(f"[case {request.param}] config {cfg} {kw}")
    w = mi.make_workload(cfg, **kw)
    g = DeviceWorkload(w, snapshot=True)
    out = g.run()
    # the first step's results (msa_decode_step from the prefix-only cache)
    g.first = dict(scores=g.step.block_scores.clone(), ids=g.step.block_ids.clone(),
                   out=out.clone(), pools=[t.clone() for t in (g.cache.k, g.cache.v, g.cache.ik)])
    return request.param, w, g, out


def test_insert_bit_exact(run):
    name, w, g, _ = run
    for b in range(w.batch):
        T = w.ctx_lens[b]
        got = gpu_sequence_caches(g.cache, w, b)
        ikc, iks = oracle.quantize(w.ik_rows(b, 0, T).numpy())
        assert np.array_equal(got["ik"][0], ikc) and np.array_equal(got["ik"][1], iks), (name, b, "ik")
        for which in ("k", "v"):
            c, s = oracle.quantize(w.kv_rows(which, b, 0, T).numpy())
            assert np.array_equal(got[which][1], s), (name, b, which, "scales")
            assert np.array_equal(got[which][0], c), (name, b, which, "codes")


def test_indexer_topk_attention(run):
    name, w, g, out = run
    exempt_total = check_step_against_oracle(w, g.step.block_scores.cpu().numpy(),
                                             g.step.block_ids.cpu().numpy(), bf16_to_f64(out))
    _log(f"[case {name}] rows below margin (validated, not bit-compared): {exempt_total}")


def test_indexer_lse_scores(run):
    # the log-sum-exp block reduction ("MiniMax M3 on vLLM", section "Prefill execution"),
    # against the oracle's: LSE is 1-Lipschitz in the token scores, so the dot-product bound
    # carries over, plus the fp32 exp / log / final-add rounding (4e-6 + 2^-22 |ref|)
    import block_sparse_attention_nvfp4_amd as msa
    name, w, g, _ = run
    q = w.q_len
    lse = torch.empty_like(g.step.block_scores)
    msa.msa_indexer_score_ex(g.cache, g.batch, g.q_idx, msa.MSA_REDUCE_LSE, lse)
    torch.cuda.synchronize()
    got = lse.cpu().numpy()
    for b in range(w.batch):
        T = w.ctx_lens[b]
        rows = slice(b * q, (b + 1) * q)
        ikc, iks = oracle.quantize(w.ik_rows(b, 0, T).numpy())
        qi = mi.bf16_bits(w.q_idx[rows])
        ref = oracle.index_scores_lse(qi, ikc, iks, T, q, w.max_blocks)
        tol = score_tolerance(qi, ikc, iks)[..., None] + 4e-6 + 2.0 ** -22 * np.abs(np.where(np.isfinite(ref), ref, 0))
        ninf = np.isneginf(ref)
        assert np.array_equal(np.isneginf(got[rows]), ninf), (name, b)
        d = np.where(ninf, 0, np.abs(got[rows].astype(np.float64) - np.where(ninf, 0, ref)))
        assert (d <= tol).all(), (name, b, float(d.max()))


def test_attention_other_scales(run):
    """Attention with softmax scales other than 1/sqrt(128), a negative one included, over the
    step's own selection (first sequence, up to four query tokens), against the oracle."""
    import block_sparse_attention_nvfp4_amd as msa
    name, w, g, _ = run
    q = w.q_len
    ids = g.step.block_ids
    toks = list(range(min(q, 4)))
    for scale in (0.37, -0.05):
        out = torch.empty_like(g.step.out)
        msa.msa_sparse_attn_decode(g.cache, g.batch, g.q, ids, scale, out, g.step.workspace)
        torch.cuda.synchronize()
        att = bf16_to_f64(out)
        ref = oracle_sequence(w, 0, attention_tokens=toks, ids_override=ids.cpu().numpy()[:q],
                              scale=scale)
        check_attention(att[:q][toks], ref["attention"])


def test_topk_bit_exact_on_shared_scores(run):
    """The selection kernel alone, fed the oracle's scores rounded to fp32, with planted ties."""
    import block_sparse_attention_nvfp4_amd as msa
    name, w, g, _ = run
    q = w.q_len
    rng = np.random.default_rng(11)
    base = np.stack([oracle_sequence(w, b)["scores"] for b in range(w.batch)]).reshape(
        w.batch * q, 4, w.max_blocks).astype(np.float32)
    # plant exact ties and negative zeros in half of the rows
    tied = base.copy()
    for r in range(0, tied.shape[0], 2):
        for gg in range(4):
            fin = np.flatnonzero(np.isfinite(tied[r, gg]))
            if len(fin) > 2:
                tied[r, gg, fin] = np.round(tied[r, gg, fin] / 8.0) * 8.0
                tied[r, gg, fin[rng.integers(0, len(fin))]] = -0.0
    for arr in (base, tied):
        s = torch.from_numpy(arr).cuda()
        ids = torch.empty((w.batch * q, 4, 16), dtype=torch.int32, device="cuda")
        msa.msa_block_topk(s, g.batch, 16, ids)
        got = ids.cpu().numpy()
        for b in range(w.batch):
            for j in range(q):
                p = w.ctx_lens[b] - q + j
                n = min(p // 128 + 1, w.max_blocks)
                for gg in range(4):
                    want, _ = oracle.block_topk(arr[b * q + j, gg].astype(np.float64), n)
                    assert np.array_equal(got[b * q + j, gg], want), (name, b, j, gg)


def test_step_is_deterministic(run):
    name, w, g, out = run
    first = out.clone()
    ids = g.step.block_ids.clone()
    again = g.run()
    assert torch.equal(ids, g.step.block_ids)
    assert torch.equal(first, again)


def _assert_same_as_first(g, step, what):
    first = g.first
    assert torch.equal(step.block_scores, first["scores"]), (what, "scores")
    assert torch.equal(step.block_ids, first["ids"]), (what, "ids")
    assert torch.equal(step.out, first["out"]), (what, "out")
    for name, got, want in zip("k v ik".split(), (g.cache.k, g.cache.v, g.cache.ik), first["pools"]):
        assert torch.equal(got, want), (what, name, "pool bytes")


def test_step_modes_agree(run):
    """msa_decode_step (the fixture's step: insert and indexer in one launch, then selection and
    attention in one) equals the three-call and the four-call sequences bit for bit: scores, ids,
    outputs and every cache byte, each run from the same prefix-only cache."""
    import block_sparse_attention_nvfp4_amd as msa
    name, w, g, _ = run
    for mode in ("select", "separate"):
        g.restore_prefix()
        st = msa.DecodeStep(g.cache, g.batch, "cuda", mode=mode)
        st.run(g.new_slots, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q)
        torch.cuda.synchronize()
        _assert_same_as_first(g, st, (name, mode))


def test_step_over_stale_slots(run):
    """The new tokens' slots first hold other tokens' bytes (a step with other values), so the
    indexer workgroups of msa_decode_step read stale bytes wherever the insert of the same launch
    has not landed yet: the results must still equal the first step's bit for bit."""
    import block_sparse_attention_nvfp4_amd as msa
    name, w, g, _ = run
    g.restore_prefix()
    gen = torch.Generator(device="cpu").manual_seed(5)
    stale = [(torch.randn(t.shape, generator=gen) * 3.0).to(t.device) for t in (g.new_k, g.new_v, g.new_ik)]
    msa.DecodeStep(g.cache, g.batch, "cuda", mode="separate").run(g.new_slots, *stale, g.q_idx, g.q)
    torch.cuda.synchronize()
    assert not torch.equal(g.cache.ik, g.first["pools"][2]), name  # the slots do hold other bytes
    g.step.run(g.new_slots, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q)
    torch.cuda.synchronize()
    _assert_same_as_first(g, g.step, (name, "stale"))
