"""The indexer over a batch that shares a prefix ("vLLM day-0 support for MiniMax-M3.1-Flash",
section "NVFP4 MSA kernel": a shared-prefix page is dequantized once for the requests that share
it), against msa_indexer_score on the same batch (the same values) and against the oracle
(needs an MI355X).

Six sequences share the pages of their first 20 blocks and each has a suffix of its own
(ragged, one of them ending 5 tokens into its first own block); 4 query tokens each. Seeded
N(0, 1) index keys and bf16 index queries.
"""
import numpy as np
import pytest
import torch

import oracle
from msa_testlib import check_scores, score_tolerance

pytestmark = pytest.mark.gpu

P = 20           # shared blocks
Q = 4
SUFFIX = [100, 700, 1500, 5, 1300, 129]


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_shared_prefix_indexer():
    import block_sparse_attention_nvfp4_amd as msa
    rng = np.random.default_rng(21)
    B = len(SUFFIX)
    T = [P * 128 + s + Q for s in SUFFIX]
    nb = [(t + 127) // 128 for t in T]
    max_blocks = max(nb)
    own = [n - P for n in nb]
    num_pages = P + sum(own) + 3
    perm = rng.permutation(num_pages)
    table = np.full((B, max_blocks), -1, np.int32)
    table[:, :P] = perm[:P]
    off = P
    for b in range(B):
        table[b, P:nb[b]] = perm[off:off + own[b]]
        off += own[b]
    prefix = rng.standard_normal((P * 128, 128)).astype(np.float32)
    ik = [np.concatenate([prefix, rng.standard_normal((T[b] - P * 128, 128)).astype(np.float32)])
          for b in range(B)]
    cache = msa.Cache.allocate(num_pages)
    dev = "cuda"
    for b in range(B):
        t0 = 0 if b == 0 else P * 128  # the shared pages are written once
        pos = np.arange(t0, T[b])
        slots = torch.from_numpy(table[b, pos // 128].astype(np.int64) * 128 + pos % 128).to(dev)
        msa.msa_kv_insert_nvfp4(cache, slots, None, None, torch.from_numpy(ik[b][t0:]).to(dev))
    batch = msa.Batch(torch.from_numpy(table).to(dev), torch.tensor(T, dtype=torch.int32, device=dev), Q)
    qi_bits = _bf16_bits(rng.standard_normal((B * Q, 4, 128)))
    q_idx = torch.from_numpy(qi_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    plain = torch.empty((B * Q, 4, max_blocks), dtype=torch.float32, device=dev)
    shared = torch.full_like(plain, 7.0)
    msa.msa_indexer_score(cache, batch, q_idx, plain)
    msa.msa_indexer_score_shared_prefix(cache, batch, q_idx, P, shared)
    none_shared = torch.full_like(plain, 7.0)  # prefix_blocks = 0: every block per sequence
    msa.msa_indexer_score_shared_prefix(cache, batch, q_idx, 0, none_shared)
    part = torch.full_like(plain, 7.0)  # a shorter shared range than the pages allow
    msa.msa_indexer_score_shared_prefix(cache, batch, q_idx, P // 2 + 1, part)
    torch.cuda.synchronize()
    got, want = shared.cpu().numpy(), plain.cpu().numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(none_shared.cpu().numpy(), want)
    assert np.array_equal(part.cpu().numpy(), want)
    for b in (0, 3, 5):
        codes, scales = oracle.quantize(ik[b])
        qb = qi_bits[b * Q:(b + 1) * Q]
        ref = oracle.index_scores(qb, codes, scales, T[b], Q, max_blocks)
        check_scores(got[b * Q:(b + 1) * Q], ref, score_tolerance(qb, codes, scales))


# ---------------------------------------------------------------- attention over a shared prefix
def _prefix_case(q_len, batch, prefix_blocks, fill, seed):
    import block_sparse_attention_nvfp4_amd as msa
    import msa_inputs as mi
    from msa_testlib import DeviceWorkload
    w = mi.make_workload(6, batch=batch, q_len=q_len, prefix_blocks=prefix_blocks, seed=seed)
    d = DeviceWorkload(w, fill=fill)
    msa.msa_kv_insert_nvfp4(d.cache, d.new_slots, d.new_k, d.new_v, d.new_ik)
    rows = batch * q_len
    scores = torch.empty((rows, 4, w.max_blocks), dtype=torch.float32, device="cuda")
    msa.msa_indexer_score(d.cache, d.batch, d.q_idx, scores)
    ids = torch.empty((rows, 4, 16), dtype=torch.int32, device="cuda")
    msa.msa_block_topk(scores, d.batch, 16, ids)
    return w, d, scores, ids


@pytest.mark.parametrize("q_len,batch,prefix_blocks,fill", [
    (1, 12, 20, 0), (4, 6, 20, 0xFF), (1, 40, 9, 0xFF)])
def test_shared_prefix_attention_against_oracle(q_len, batch, prefix_blocks, fill):
    """Requests sharing a prefix (the seeded prefix workload at reduced size: every request's
    first blocks are the same pages, its suffix its own); the attention that dequantizes each
    selected shared block once for all rows that selected it, with the whole prefix shared, part
    of it, and none, against the oracle over the GPU's own selection (which the same call checks
    against the oracle's), and against the per-row attention within the same tolerance."""
    import block_sparse_attention_nvfp4_amd as msa
    import msa_inputs as mi
    from msa_testlib import check_attention, check_step_against_oracle, oracle_sequence
    w, d, scores, ids = _prefix_case(q_len, batch, prefix_blocks, fill, seed=60 + q_len)
    rows = batch * q_len
    scale = msa.default_softmax_scale()
    ws = torch.empty(msa.msa_sparse_attn_shared_prefix_workspace_bytes(d.batch), dtype=torch.uint8,
                     device="cuda")
    outs = {}
    for p in (prefix_blocks, prefix_blocks // 2 + 1, 0):
        out = torch.full((rows, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        msa.msa_sparse_attn_decode_shared_prefix(d.cache, d.batch, d.q, ids, p, scale, out, ws)
        outs[p] = out
    plain = torch.empty((rows, 64, 128), dtype=torch.bfloat16, device="cuda")
    need = msa.msa_sparse_attn_workspace_bytes(d.batch)
    pws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    msa.msa_sparse_attn_decode(d.cache, d.batch, d.q, ids, scale, plain, pws if need else None)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    # the shared path is exercised: some shared block is selected by several rows of a group
    sel = ids_h[(ids_h >= 0) & (ids_h < prefix_blocks)]
    assert sel.size > 0
    counts = [np.bincount(ids_h[:, g][(ids_h[:, g] >= 0) & (ids_h[:, g] < prefix_blocks)],
                          minlength=prefix_blocks) for g in range(4)]
    assert max(c.max() for c in counts) >= 2
    s_h = scores.cpu().numpy()
    check_step_against_oracle(w, s_h, ids_h, outs[prefix_blocks].float().cpu().numpy())
    got = {p: o.float().cpu().numpy().astype(np.float64) for p, o in outs.items()}
    got["plain"] = plain.float().cpu().numpy().astype(np.float64)
    for b in range(batch):
        r = slice(b * q_len, (b + 1) * q_len)
        ref = oracle_sequence(w, b, attention_tokens=list(range(q_len)), ids_override=ids_h[r])
        for key, g in got.items():
            check_attention(g[r], ref["attention"])
