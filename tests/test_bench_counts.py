"""CPU checks of the work bench.py divides by: masked FLOPs and visible
pairs of the measured layers (closed forms and the oracle's masks)."""
import numpy as np

import bench
import oracle
import workloads as W


def test_masked_flops_of_the_measured_layers():
    # 4 chunks of 1440 tokens: pairs per head = 1440^2 (1 + 2 + 3 + 4)
    assert bench.masked_flops(W.make_workload("magi4.5b")) == 4 * 24 * 128 * 1440 ** 2 * 10
    # 8 chunks of 3600 tokens: 3600^2 (1 + ... + 8)
    assert bench.masked_flops(W.make_workload("magi24b")) == 4 * 48 * 128 * 3600 ** 2 * 36


def test_visible_pairs_match_the_oracle_mask():
    wl = W.make_workload("tiny")
    assert bench.visible_pairs(wl) == int(oracle.video_mask(wl.seqs, wl.nq, wl.nk).sum())
    wl = W.custom_packed([(3, 1, 3, 4, [-1, 1, -1]), (2, 2, 2, 3, None)], 8, 2, 24)
    assert bench.visible_pairs(wl) == int(oracle.video_mask(wl.seqs, wl.nq, wl.nk).sum())


def test_window_pairs_match_the_oracle_mask():
    wl = W.custom_packed([(3, 1, 3, 4, None), (2, 2, 2, 3, None)], 8, 2, 24)
    for w in (1, 5, 12, 40):
        spec = [(s.num_q_chunks * s.chunk_len, w, s.q_offset, s.k_offset) for s in wl.seqs]
        assert bench.window_pairs(wl, w) == int(oracle.window_mask(spec, wl.nq, wl.nk).sum())
