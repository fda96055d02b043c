"""msa_decode_step_noalloc (the decode step with the library's static workspace) against
msa_decode_step with a caller-owned workspace, through the C ABI (needs an MI355X).

Two calls in a row, the second with a smaller batch: every output (block scores, selected ids,
attention outputs) and every cache byte must equal the workspace call's bit for bit (the same
kernels run on the same inputs), and the outputs must also match the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import msa_inputs as mi
from msa_testlib import DeviceWorkload, bf16_to_f64, check_step_against_oracle

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_step_equals_workspace_step():
    import block_sparse_attention_nvfp4_amd as msa
    # the first call needs 2 splits per row group (512 rows: 8.7 MB of the static array), the
    # second is smaller (12 rows, 4 splits) and reuses the array the first left behind
    for cfg, kw in ((3, dict(batch=32, ctx=3000, q_len=4)), (2, dict(batch=3, ctx=2500, q_len=1))):
        _log(f"[noalloc] config {cfg} {kw}")
        w = mi.make_workload(cfg, **kw)
        g = DeviceWorkload(w, snapshot=True)
        assert msa.msa_sparse_attn_workspace_bytes(g.batch) > 0  # the split path runs
        ref_out = g.run().clone()
        ref = dict(scores=g.step.block_scores.clone(), ids=g.step.block_ids.clone(),
                   pools=[t.clone() for t in (g.cache.k, g.cache.v, g.cache.ik)])
        g.restore_prefix()
        scores = torch.full_like(ref["scores"], float("nan"))
        ids = torch.full_like(ref["ids"], -7)
        out = torch.full_like(ref_out, float("nan"))
        msa.msa_decode_step_noalloc(g.cache, g.batch, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q, 16,
                                    msa.default_softmax_scale(), scores, ids, out)
        torch.cuda.synchronize()
        assert torch.equal(scores, ref["scores"]), "block scores differ"
        assert torch.equal(ids, ref["ids"]), "selected ids differ"
        assert torch.equal(out, ref_out), "attention outputs differ"
        for name, got, want in zip("k v ik".split(), (g.cache.k, g.cache.v, g.cache.ik), ref["pools"]):
            assert torch.equal(got, want), (name, "pool bytes differ")
        check_step_against_oracle(w, scores.cpu().numpy(), ids.cpu().numpy(), bf16_to_f64(out),
                                  max_tokens=4)
        _log(f"[noalloc] config {cfg} ok")
