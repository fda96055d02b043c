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
