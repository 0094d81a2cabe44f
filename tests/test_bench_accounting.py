"""bench.py's host-side accounting (CPU): the run structure it reads back
from the metadata, the hot-row plan's choice it replays to split the long
runs between the matrix-core contraction and the chunk path, and the byte
and flop models built on them. The metadata comes from the oracle's own
preprocessing of a small skewed batch; the expected values are computed
here independently, run by run."""
import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import LARGE, make_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _meta(cfg, batch, S, C):
    pre = oracle.preprocess(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets, batch.psw, S, C)
    U = int(pre["U"])
    ro = pre["run_offsets"][:U + 1].astype(np.int64)
    sl = np.diff(ro)
    counts = [U, int((sl < S).sum()), int((sl >= S).sum()),
              int(((sl[sl >= S] + C - 1) // C).sum())]
    meta = {"counts": torch.tensor(counts), "run_offsets": torch.from_numpy(ro),
            "sorted_bag": torch.from_numpy(pre["sorted_bag"].astype(np.int64)),
            "run_keys": torch.from_numpy(pre["run_keys"][:U].astype(np.int64))}
    return pre, meta, sl


def _hot_runs(cfg, run_keys, sl, S, K):
    """Per table, the long runs of at least v lookups, v the least length that
    leaves at most K of them (a tie at the cut leaves every tied run out)."""
    toff = np.concatenate([[0], np.cumsum(cfg.rows)])
    table = np.searchsorted(toff, run_keys, side="right") - 1
    hot = np.zeros(sl.size, dtype=bool)
    for t in range(cfg.T):
        mine = np.nonzero((table == t) & (sl >= S))[0]
        lens = sl[mine]
        for v in range(S, int(lens.max(initial=S)) + 2):
            if (lens >= v).sum() <= K:
                hot[mine[lens >= v]] = True
                break
    return hot


@pytest.mark.parametrize("K", [256, 8])
def test_run_structure_replays_the_hot_plan(bench, K, monkeypatch):
    """With the default K every long run of this small batch is hot; with
    K = 8 the choice cuts inside each table, ties included."""
    monkeypatch.setattr(bench, "HOT_K", K)
    cfg = LARGE
    batch = make_batch(cfg, B=2048)
    c = batch.cfg
    S, C = 64, 64
    pre, meta, sl = _meta(c, batch, S, C)
    st = bench.run_structure(torch, meta, c, batch.indices.size, S=S, C=C, hot=True)
    hot = _hot_runs(c, pre["run_keys"][:sl.size], sl, S, K)
    long_ = sl >= S
    assert st["long_lookups"] == int(sl[long_].sum())
    assert st["hot_runs"] == int(hot.sum())
    assert st["hot_lookups"] == int(sl[hot].sum())
    rest = long_ & ~hot
    assert st["chunk_chunks"] == int(((sl[rest] + C - 1) // C).sum())
    # bags that some lookup of a remaining long run falls in
    bags = pre["sorted_bag"][np.repeat(rest, sl)]
    assert st["bags_chunk"] == np.unique(bags).size
    if K == 8:
        assert 0 < st["hot_runs"] < int(long_.sum())


def test_byte_and_flop_models_with_the_contraction(bench):
    cfg = LARGE
    batch = make_batch(cfg, B=2048)
    c = batch.cfg
    S, C = 64, 64
    pre, meta, sl = _meta(c, batch, S, C)
    N = batch.indices.size
    st0 = bench.run_structure(torch, meta, c, N, S=S, C=C, hot=False)
    st1 = bench.run_structure(torch, meta, c, N, S=S, C=C, hot=True)
    b0 = bench.compulsory_bytes(c, st0, True)
    b1 = bench.compulsory_bytes(c, st1, True)
    # the forward and the short runs do not change; the contraction reads
    # every gradient row, index and weight once and writes its partials
    assert b0["fwd"] == b1["fwd"] and b0["bwd_short"] == b1["bwd_short"]
    parts = 4 * c.T * st1["hot_nseg"] * 256 * c.D
    assert b1["bwd_hot"] == c.T * c.B * 4 * c.D + N * 8 + 4 * (c.T * c.B + 1) + parts
    assert "bwd_hot" not in b0
    # segments: at most 512 workgroups over all tables, at least 32 tiles each
    tiles = -(-c.B // 16)
    assert st1["hot_nseg"] == max(1, min(512 // c.T, -(-tiles // 32)))
    # flops: three products of 256 slots x 16 bags x D per 16-bag tile
    assert bench.hot_flops(c, st1, True) == 2 * 3 * c.T * tiles * 16 * 256 * c.D
    assert bench.hot_flops(c, st1, False) == 2 * 2 * c.T * tiles * 16 * 256 * c.D
