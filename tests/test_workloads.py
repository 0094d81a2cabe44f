"""The seeded generator reproduces the workload statistics the pages state."""
import json
import os

import numpy as np
import pytest
import torch

from workloads import WORKLOADS, TINY, DEMO3, MEDIUM, LARGE, SMALL_TABLE, init_state, init_weights, make_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.slow
def test_large_config_matches_page_index_statistics():
    g = json.load(open(os.path.join(GOLDEN, "page1_index_stats.json")))
    cfg = LARGE
    assert cfg.T * cfg.B == g["T_times_B"] and cfg.B == g["B"]
    b = make_batch(cfg, with_grad=False)
    first = np.arange(cfg.T, dtype=np.int64) * cfg.rows[0]
    t_of = np.repeat(np.arange(cfg.T), np.diff(b.offsets[::cfg.B]))
    keys = first[t_of] + b.indices
    counts = np.bincount(keys, minlength=cfg.sum_rows)
    tol = g["relative_tolerance"]
    assert abs(b.N / g["lookups"] - 1) < tol
    assert abs(np.count_nonzero(counts) / g["unique_rows"] - 1) < tol
    assert abs(counts.max() / g["max_row_frequency"] - 1) < tol


def test_batch_layout_and_determinism():
    for cfg in (TINY, DEMO3, MEDIUM, SMALL_TABLE):
        b1 = make_batch(cfg, B=64)
        b2 = make_batch(cfg, B=64)
        assert np.array_equal(b1.indices, b2.indices) and np.array_equal(b1.grad, b2.grad)
        assert b1.offsets.dtype == np.int32 and b1.offsets[0] == 0
        assert b1.offsets.size == cfg.T * 64 + 1 and b1.offsets[-1] == b1.indices.size
        assert np.all(np.diff(b1.offsets) >= 0)
        assert b1.grad.shape == (64, cfg.T * cfg.D) and b1.grad.dtype == np.float32
        for t in range(cfg.T):
            a, e = b1.offsets[t * 64], b1.offsets[(t + 1) * 64]
            seg = b1.indices[a:e]
            assert seg.size == 0 or (seg.min() >= 0 and seg.max() < cfg.rows[t])


def test_bag_length_distributions():
    b = make_batch(DEMO3, B=4096, with_grad=False)
    L = np.diff(b.offsets).reshape(3, 4096)
    assert np.all(L[0] == 1) and L[1].min() >= 1 and L[1].max() <= 20
    b5 = make_batch(SMALL_TABLE, B=128, with_grad=False)
    assert np.all(np.diff(b5.offsets) == 64)


def test_weights_and_state_are_seeded_and_in_range():
    cfg = TINY
    w1 = init_weights(cfg, "cpu", chunk_rows=300)
    w2 = init_weights(cfg, "cpu", chunk_rows=300)
    assert w1.dtype == torch.float32 and w1.shape == (2000, 16) and torch.equal(w1, w2)
    assert w1.abs().max() <= 0.01 and w1.std() > 0.004
    w16 = init_weights(SMALL_TABLE, "cpu")
    assert w16.dtype == torch.float16 and w16.shape == (64 * 64, 128)
    m = init_state(cfg, "cpu", m0="uniform")
    assert m.min() >= 0 and m.max() < 1 and m.unique().numel() > 1900
    assert not init_state(cfg, "cpu").any()
