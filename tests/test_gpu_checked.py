"""The checked build of the library (libmsa_checked.so, include/msa_debug.h) on the GPU.

The same sources compiled with MSA_CHECKED count failed checks of the values the kernels read
from device memory (context lengths) and of their own index arithmetic (selections ascending
within the eligible blocks with the query token's block last, split partials within the
workspace, list and table indexes within their on-chip arrays, row indexes within their arrays).
On workloads that keep every contract the checked build must count no failure and give the
normal build's results bit for bit; a context length past the block table's capacity, which
every build clamps, must be counted at its site (MSA_CHECK_CTX_LEN) without changing what the
kernels touch.
"""
import sys

import pytest
import torch

import msa_inputs as mi
from msa_testlib import DeviceWorkload

pytestmark = pytest.mark.gpu

MSA_CHECK_CTX_LEN = 1


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# every step mode on each: the decode kernels (per-token attention with 4 and 2 splits and the
# fused selection, the union kernel, rows past 1,025 and past 2,048 blocks), and the prefill
# kernels (score-GEMM
# indexer, token tiles over 1,024 rows, run insert)
CASES = {
    "spec_q4": (3, dict(batch=2, ctx=6000)),
    "batched_q1": (2, dict(batch=3, ctx=9000)),
    "ragged": (4, dict(batch=5, ctx_lens=[3000, 129, 7777, 17 * 128 + 5, 2048])),
    "two_splits": (2, dict(batch=130, ctx=1500, q_len=1)),
    "union_q4": (3, dict(batch=16, ctx=2600)),
    "long_rows": (4, dict(batch=2, ctx_lens=[140_001, 2_000])),
    "long_table": (4, dict(batch=2, ctx_lens=[2100 * 128 + 77, 2_000])),
    "prefill": (5, dict(batch=1, ctx=2048 + 256, q_len=256)),
}


def _step_results(msa, g, mode):
    g.restore_prefix()
    st = msa.DecodeStep(g.cache, g.batch, "cuda", mode=mode)
    st.run(g.new_slots, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q)
    torch.cuda.synchronize()
    return [st.block_scores.clone(), st.block_ids.clone(), st.out.clone(),
            *(t.clone() for t in (g.cache.k, g.cache.v, g.cache.ik))]


@pytest.mark.parametrize("name", list(CASES))
def test_checked_build_counts_nothing_and_matches(name):
    import block_sparse_attention_nvfp4_amd as msa
    cfg, kw = CASES[name]
    _log(f"checked build case {name}: config {cfg} {kw}")
    w = mi.make_workload(cfg, **kw)
    g = DeviceWorkload(w, snapshot=True)
    try:
        for mode in ("step", "select", "separate"):
            msa.use_library(False)
            want = _step_results(msa, g, mode)
            msa.use_library(True)
            msa.msa_debug_checks()  # counters reset before the run
            got = _step_results(msa, g, mode)
            assert msa.msa_debug_checks() == (0, 0), (name, mode)
            for i, (a, b) in enumerate(zip(got, want)):
                assert torch.equal(a, b), (name, mode, i)
    finally:
        msa.use_library(False)


def test_checked_build_counts_a_context_past_the_table():
    """Sequence 1's context length is set past its block table's capacity (max_blocks * 128
    tokens); every kernel clamps it, and the checked build reports the clamp at its site. The
    other sequence's results are those of the normal build, bit for bit."""
    import block_sparse_attention_nvfp4_amd as msa
    _log("checked build: context length past the table")
    w = mi.make_workload(3, batch=2, ctx=5000, q_len=4, seed=61)
    g = DeviceWorkload(w, snapshot=True)
    cap = w.max_blocks * 128
    bad = g.ctx.clone()
    bad[1] = cap + 77
    try:
        results = {}
        for checked in (False, True):
            msa.use_library(checked)
            if checked:
                msa.msa_debug_checks()
            g.restore_prefix()
            g.ctx.copy_(bad)
            st = msa.DecodeStep(g.cache, g.batch, "cuda", mode="step")
            st.run(g.new_slots, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q)
            torch.cuda.synchronize()
            results[checked] = (st.block_scores.clone(), st.block_ids.clone(), st.out.clone())
            if checked:
                count, site = msa.msa_debug_checks()
                assert count > 0 and site == MSA_CHECK_CTX_LEN, (count, site)
                assert msa.msa_debug_checks() == (0, 0)  # read and reset
        q = w.q_len
        for a, b in zip(results[True], results[False]):
            assert torch.equal(a[:q], b[:q])  # sequence 0's rows
            assert torch.equal(a, b)  # the clamp is the same in both builds
    finally:
        msa.use_library(False)
