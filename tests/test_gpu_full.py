"""HIP path vs the oracle at the five workloads' full sizes (needs an MI355X).

Each workload runs through the same DecodeStep launches the benchmark times (insert of the
step's new tokens, indexer, top-k, attention and, when split, the merge). The oracle then checks:

* quantization bit for bit on sampled blocks of every sequence (first, a middle one, the last,
  which holds the new tokens and, where ragged, the partial tail);
* index scores within the fp32 accumulation bound and selections bit for bit, on every row
  of the decode workloads and on sampled rows of the prefill chunk (each scored on its own
  causal prefix, which is all the oracle needs for one row);
* attention within |d| <= 2e-3 + 1e-2 |ref| per element and 1e-2 relative L2 on sampled rows.

Sequences use the retry counters of tests/golden/retries.json, so that every selection row has
an oracle margin of at least 1e-3 and the selections can be compared exactly.
"""
import sys

import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from msa_testlib import (DeviceWorkload, bf16_to_f64, check_attention, check_scores, check_selection,
                         gpu_block_caches, oracle_rows, score_tolerance)

pytestmark = pytest.mark.gpu

CONFIGS = [1, 2, 3, 4, 5]
PREFILL_ROWS = [0, 1, 127, 128, 1000, 2047]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=CONFIGS, ids=lambda c: mi.CONFIGS[c]["name"])
def full(request):
    cfg = request.param
    w = mi.full_workload(cfg)
    _log(f"[full {w.name}] batch {w.batch} q_len {w.q_len} ctx {w.ctx_lens} pages {w.num_pages}")
    g = DeviceWorkload(w)
    out = g.run()
    _log(f"[full {w.name}] step done")
    yield cfg, w, g, out
    del g
    torch.cuda.empty_cache()


def _rows(w):
    return list(range(w.q_len)) if w.q_len <= 8 else PREFILL_ROWS


def test_full_insert_sampled_blocks(full):
    cfg, w, g, _ = full
    for b in range(w.batch):
        nb = w.n_blocks(b)
        blocks = sorted({0, nb // 2, nb - 1})
        got = gpu_block_caches(g.cache, w, b, blocks)
        T = w.ctx_lens[b]
        for name in ("ik", "k", "v"):
            want_c, want_s = [], []
            for blk in blocks:
                t0, t1 = blk * 128, min(T, blk * 128 + 128)
                x = (w.ik_rows if name == "ik" else (lambda bb, a, z: w.kv_rows(name, bb, a, z)))(b, t0, t1)
                c, s = oracle.quantize(x.numpy())
                want_c.append(c)
                want_s.append(s)
            # compare the valid tokens of each block (slots past T were never written)
            off = 0
            for blk, c, s in zip(blocks, want_c, want_s):
                n = len(c)
                gc = got[name][0][off:off + n]
                gs = got[name][1][off:off + n]
                assert np.array_equal(gs, s), (w.name, b, blk, name, "scales")
                assert np.array_equal(gc, c), (w.name, b, blk, name, "codes")
                off += 128


def test_full_scores_and_selection(full):
    cfg, w, g, _ = full
    q = w.q_len
    scores = g.step.block_scores.cpu().numpy()
    ids = g.step.block_ids.cpu().numpy()
    rows = _rows(w)
    worst = 0.0
    for b in range(w.batch):
        T = w.ctx_lens[b]
        ref = oracle_rows(w, b, rows, attention=False)
        got_s = scores[b * q:(b + 1) * q][rows]
        got_i = ids[b * q:(b + 1) * q][rows]
        qi = mi.bf16_bits(w.q_idx[b * q:(b + 1) * q])[rows]
        tol = score_tolerance(qi, *ref["ik"])
        worst = max(worst, check_scores(got_s, ref["scores"], tol))
        for i, j in enumerate(rows):
            # the row-by-row oracle scores each token on its own prefix: same selection rule
            p = T - q + j
            exempt = check_selection(got_i[i:i + 1], ref["ids"][i:i + 1], ref["margins"][i:i + 1],
                                     ref["scores"][i:i + 1], tol[i:i + 1], p + 1, 1)
            assert exempt == 0, (w.name, b, j, "row below the 1e-3 margin despite retries")
    _log(f"[full {w.name}] scores worst |d| {worst:.3e}; {w.batch * len(rows) * 4} selections exact")


def test_full_attention_sampled(full):
    cfg, w, g, out = full
    q = w.q_len
    ids = g.step.block_ids.cpu().numpy()
    rows = _rows(w)
    seqs = range(w.batch) if w.batch <= 8 else [0, 1, w.batch // 2, w.batch - 1]
    att = bf16_to_f64(out)
    worst = 0.0
    for b in seqs:
        sel = ids[b * q:(b + 1) * q][rows]
        ref = oracle_rows(w, b, rows, ids_override=sel)
        d, _ = check_attention(att[b * q:(b + 1) * q][rows], ref["attention"])
        worst = max(worst, d)
    _log(f"[full {w.name}] attention worst |d| {worst:.3e}")
