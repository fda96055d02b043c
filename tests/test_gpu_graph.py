"""A decode step captured in a HIP graph gives the eager result on every replay (needs a GPU).

The step's launches have shape-stable grids and issue no memset, so the whole four-call step
can be captured ("MiniMax M3 on vLLM", section "Speculative decoding in the decode kernels":
shape-stable launch grids make the decode path safe for graph replay).
"""
import pytest
import torch

import msa_inputs as mi
from msa_testlib import DeviceWorkload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,kw", [(3, dict(batch=2, ctx=6000)), (2, dict(batch=3, ctx=9000)),
                                    (5, dict(batch=1, ctx=2048 + 64, q_len=64))])
def test_graph_replays_match_eager(cfg, kw):
    print(f"[graph] config {cfg} {kw}", flush=True)
    w = mi.make_workload(cfg, **kw)
    g = DeviceWorkload(w)
    eager_out = g.run().clone()
    eager_ids = g.step.block_ids.clone()
    eager_scores = g.step.block_scores.clone()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        g.step.run(g.new_slots, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q)  # warm on the stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            g.step.run(g.new_slots, g.new_k, g.new_v, g.new_ik, g.q_idx, g.q)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays that overwrites the step's outputs
        g.step.out.zero_()
        g.step.block_ids.fill_(-7)
        g.step.block_scores.fill_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g.step.block_scores, eager_scores), rep
        assert torch.equal(g.step.block_ids, eager_ids), rep
        assert torch.equal(g.step.out, eager_out), rep
