"""Host checks of the seeded input generator: determinism, slice independence, structure."""
import math

import numpy as np
import torch

import msa_inputs as mi


def test_draw_is_deterministic_and_sliceable():
    key = mi.stream_key(3, mi.TAG_IK, 5, 0)
    a = mi.draw("normal", key, 0, 10000)
    b = mi.draw("normal", key, 0, 10000)
    assert torch.equal(a, b)
    assert torch.equal(a[4000:7000], mi.draw("normal", key, 4000, 3000))
    other = mi.draw("normal", mi.stream_key(3, mi.TAG_IK, 6, 0), 0, 10000)
    assert not torch.equal(a, other)


def test_pool_moments():
    x = mi.draw("normal", mi.stream_key(1, 1), 0, 1 << 20).double()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1) < 0.01
    t = mi.draw("t3", mi.stream_key(1, 2), 0, 1 << 20).double()
    assert abs(t.median().item()) < 0.01
    assert t.abs().max().item() > 10          # heavy tails


def test_workload_structure_configs():
    for cfg in (1, 2, 3, 4, 5):
        w = mi.make_workload(cfg)
        full = mi.CONFIGS[cfg]
        assert w.batch == full["batch"] and w.q_len == full["q_len"]
        used = w.block_table[w.block_table >= 0]
        assert len(np.unique(used)) == len(used) == w.num_pages   # a permutation of the pool
        for b in range(w.batch):
            nb = w.n_blocks(b)
            assert np.all(w.block_table[b, :nb] >= 0) and np.all(w.block_table[b, nb:] == -1)
        assert w.q_idx.shape == (w.batch * w.q_len, 4, 128) and w.q_idx.dtype == torch.bfloat16
        assert w.q.shape == (w.batch * w.q_len, 64, 128) and w.q.dtype == torch.bfloat16
    w1 = mi.make_workload(1)
    assert np.array_equal(w1.block_table[0], np.arange(32))
    w4 = mi.make_workload(4)
    assert all(8192 <= t <= 524288 and t % 128 != 0 for t in w4.ctx_lens)
    assert w4.plants == {}
    w3 = mi.make_workload(3)
    assert all(len(v) == 16 and all(1.5 <= a <= 3.0 for _, a in v) for v in w3.plants.values())
    w5 = mi.make_workload(5)
    assert all(len(v) == 15 and all(b < 512 for b, _ in v) for v in w5.plants.values())


def test_planting_adds_alpha_w_before_quantization():
    w = mi.make_workload(1)
    (blk, alpha), = w.plants[(0, 2)][:1]
    base_key = mi.stream_key(w.seed, mi.TAG_IK, 0, 0)
    noise = mi.draw("normal", base_key, blk * 128 * 128, 128 * 128).view(128, 128)
    rows = w.ik_rows(0, blk * 128, blk * 128 + 128)
    shift = torch.zeros(128)
    for g in range(4):
        for b2, a2 in w.plants[(0, g)]:
            if b2 == blk:
                shift = shift + torch.from_numpy(np.float32(a2) * w.plant_dir[0, g])
    assert torch.allclose(rows, noise + shift, rtol=0, atol=1e-5)
    assert w.plant_dir.shape == (1, 4, 128)


def test_retry_redraws_only_that_sequence():
    a = mi.make_workload(2, batch=3, ctx=1024)
    b = mi.make_workload(2, batch=3, ctx=1024, retries={1: 2})
    assert torch.equal(a.ik_rows(0, 0, 256), b.ik_rows(0, 0, 256))
    assert not torch.equal(a.ik_rows(1, 0, 256), b.ik_rows(1, 0, 256))
    assert a.plants[(0, 1)] == b.plants[(0, 1)]


def test_prefix_workload_shares_pages_and_data():
    """The prefix-sharing workload: every request's first blocks are the same pages holding the
    same data, the suffixes are the requests' own (own pages, own data), the query tokens lie
    past the prefix, the planted blocks and the index-query direction are the batch's."""
    w = mi.make_workload(6, batch=5, prefix_blocks=7)
    P = 7
    assert w.prefix_tokens == P * 128
    assert (w.block_table[:, :P] == w.block_table[0, :P]).all()
    own = [set(w.block_table[b, P:w.n_blocks(b)].tolist()) for b in range(w.batch)]
    assert all(-1 not in s for s in own)
    for a in range(w.batch):
        assert not own[a] & set(w.block_table[0, :P].tolist())
        for b in range(a + 1, w.batch):
            assert not own[a] & own[b]
    used = w.block_table[w.block_table >= 0]
    assert len(np.unique(used)) == w.num_pages
    for b in range(1, w.batch):
        assert torch.equal(w.ik_rows(b, 0, P * 128), w.ik_rows(0, 0, P * 128))
        assert torch.equal(w.kv_rows("v", b, 100, P * 128 + 50)[: P * 128 - 100],
                           w.kv_rows("v", 0, 100, P * 128))
        assert not torch.equal(w.ik_rows(b, P * 128, P * 128 + 64), w.ik_rows(0, P * 128, P * 128 + 64))
        assert w.plants[(b, 2)] == w.plants[(0, 2)]
        assert all(blk < P for blk, _ in w.plants[(b, 2)])
    assert all(T - w.q_len >= P * 128 and T % 128 != 0 for T in w.ctx_lens)
    assert np.array_equal(w.plant_dir[0], w.plant_dir[3])
