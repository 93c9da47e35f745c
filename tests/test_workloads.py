"""Host checks of the seeded workload descriptions and input draws."""
import numpy as np
import torch

import workloads as W


def test_shapes_of_the_five_workloads():
    t = W.make_workload("tiny")
    assert (t.nq, t.nk, t.hq, t.hkv, t.head_dim, t.dtype) == (144, 144, 8, 2, 24, "fp32")
    a = W.make_workload("magi4.5b")
    assert (a.nq, a.seqs[0].chunk_len, a.hq, a.hkv, a.head_dim) == (5760, 1440, 128, 8, 24)
    b = W.make_workload("magi24b")
    assert (b.nq, b.seqs[0].chunk_len, b.head_dim) == (28800, 3600, 48)
    s = W.make_workload("stream")
    assert (s.nq, s.nk, s.k_fresh_start) == (14400, 86400, 72000)
    v = W.make_workload("varlen", 0)
    assert [x.num_kv_chunks for x in v.seqs] == [6, 15, 5, 5, 12, 11]
    assert sum(r == 3 for x in v.seqs for r in x.kv_range) == 10
    assert v.nq == v.nk == 54 * 2400


def test_varlen_plan_limits_only_late_chunks():
    for seed in range(5):
        counts, limited = W.varlen_chunk_plan(seed)
        assert sum(counts) == 54 and all(2 <= c <= 16 for c in counts)
        assert all(not f for fl in limited for f in fl[:4])


def test_token_coords_layout():
    wl = W.custom_block_causal(3, 2, 2, 3, 4, 2, 24)
    pq, pk = W.token_coords(wl)
    np.testing.assert_array_equal(pq, pk)
    # chunk 1, frame 1, row 1, col 2 -> token 12 + 6 + 3 + 2
    np.testing.assert_array_equal(pq[12 + 6 + 3 + 2], [1 * 2 + 1, 1, 2])
    s = W.make_workload("stream")
    pq, pk = W.token_coords(s)
    assert pq[0, 0] == 20 * 6 and pk[-1, 0] == 24 * 6 - 1


def test_inputs_are_reproducible_and_rowwise():
    wl = W.custom_block_causal(2, 2, 4, 4, 8, 2, 24)
    a = W.make_inputs(wl, 3)
    b = W.make_inputs(wl, 3)
    assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v)
    rows = np.array([0, 5, 31, 63])
    c = W.make_inputs(wl, 3, q_rows=rows)
    assert torch.equal(c.q, a.q[rows]) and torch.equal(c.pos_q, a.pos_q[rows])
    assert a.q.dtype == torch.bfloat16
    # bf16 values are the round-to-nearest-even images of the float32 draws
    raw = W._draw_normal(3, 1, wl.nq, wl.hq * 24).reshape(wl.nq, wl.hq, 24)
    assert torch.equal(torch.from_numpy(raw).to(torch.bfloat16), a.q)
    assert float(a.gain_q.min()) >= 0.8 and float(a.gain_q.max()) <= 1.2
