"""Backward of the hot rows (the rows of each table's longest runs) on the
matrix cores (TBE_FLAG_HOT_BACKWARD), through the C ABI against the oracle. Each gradient row is read
once per table and contracted with the hot rows' per-bag weight sums; the
other long runs keep the chunk path and the apply sums a hot row's segment
partials. Every updated row must match the oracle (weights within tolerance
and 1 ulp of the rounded oracle, state within 1e-5), untouched rows stay
bitwise unchanged, and the stage timer shows the contraction ran. Covered:
weighted bf16 and unweighted f16, rows of 32, 64, 96 and 128, more long runs
than the 256 hot slots, runs tied at the cut (no hot row), a ragged last
segment, bags longer than the lookups staged ahead, and scales moved by later
tiles: one gradient far above its column's scale, and every segment's first
tile 1e-6 times smaller than the rest; hot rows above 2^23 in a table of
2^24 - 2 rows (the largest the packed row-and-slot hash takes), and a table
of 2^24 - 1 rows, which leaves every hot run to the chunk path."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import (assert_rows_match, assert_untouched_unchanged, fresh_params,
                              host_rows, oracle_all, run_library)
from workloads import LARGE, Batch, Config, make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401


def _check(cfg, batch, S=0, C=0, label="", hot=True):
    import bwd_tbe_pooled_amd as tbe
    print(f"\n[hotbwd] {label or cfg.name} T={cfg.T} B={cfg.B} D={cfg.D} {cfg.dtype} "
          f"N={batch.indices.size} S={S or 256}", flush=True)
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W0, m0, uk)
    timer = tbe.Timer(4)
    r = run_library(cfg, batch, W, m, meta_in_forward=True, S=S, C=C, timer=timer,
                    flags=tbe.TBE_FLAG_HOT_BACKWARD)
    pre, _, bw = oracle_all(cfg, batch, Wrows, mrows, uk, S or 256, C or 256)
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"], label or cfg.name)
    assert_untouched_unchanged(W0, W, m0, m, uk)
    if hot:
        assert timer.read()["bwd_hot"][1] == 1, "the hot rows' contraction did not run"
    else:
        assert timer.read()["bwd_hot"][1] == 0, "the hot rows' contraction ran"
    return pre


def test_more_long_runs_than_hot_slots_weighted_bf16():
    """600 rows per table, every one a long run (S = 16): the 256 longest
    take the contraction, the rest the chunk path."""
    cfg = Config("hot_many", T=4, B=4096, D=128, rows=(600,) * 4, dtype="bf16",
                 bag=("fixed", 20), index=("uniform",), weighted=True,
                 preprocess_in_forward=True, seed=81)
    pre = _check(cfg, make_batch(cfg), S=16, C=64)
    assert pre["long_runs"].size == 2400


@pytest.mark.parametrize("D", [32, 64, 96, 128])
def test_unweighted_f16_row_widths(D):
    cfg = Config(f"hot_f16_d{D}", T=3, B=3000, D=D, rows=(5000, 800, 20000), dtype="f16",
                 bag=("poisson", 20.0), index=("zipf", 1.1), weighted=False,
                 preprocess_in_forward=True, seed=83 + D)
    _check(cfg, make_batch(cfg), S=64, C=32)


def test_large_skewed_reduced_batch():
    batch = make_batch(LARGE, B=4096)
    _check(batch.cfg, batch, label="large skewed B=4096")


def test_ragged_last_segment():
    """64 tables of 2088 bags (131 tiles of 16, the last one of 8 bags): 5
    segments of 27 tiles per table, the last one 23 tiles long."""
    cfg = Config("hot_ragged_seg", T=64, B=2088, D=64, rows=(200,) * 64, dtype="bf16",
                 bag=("fixed", 20), index=("zipf", 1.2), weighted=True,
                 preprocess_in_forward=True, seed=85)
    _check(cfg, make_batch(cfg), S=16, C=16)


def _tied_batch(counts_per_row, B, L, seed):
    """One table whose row r appears counts_per_row[r] times, shuffled into B
    bags of L lookups, with weights and a gradient."""
    rng = np.random.default_rng(seed)
    rows = np.repeat(np.arange(len(counts_per_row)), counts_per_row)
    assert rows.size == B * L
    idx = rng.permutation(rows).astype(np.int32)
    offsets = (np.arange(B + 1, dtype=np.int32) * L).astype(np.int32)
    cfg = Config("hot_ties", T=1, B=B, D=64, rows=(len(counts_per_row),), dtype="bf16",
                 bag=("fixed", L), index=("uniform",), weighted=True,
                 preprocess_in_forward=True, seed=seed)
    psw = rng.uniform(0.5, 1.5, size=idx.size).astype(np.float32)
    grad = rng.standard_normal((B, cfg.D)).astype(np.float32)
    return cfg, Batch(cfg=cfg, indices=idx, offsets=offsets, psw=psw, grad=grad)


def test_runs_tied_at_the_cut():
    """300 runs of exactly 40 lookups: 256 slots cannot take a length, so no
    run of the table is hot and all take the chunk path."""
    cfg, batch = _tied_batch([40] * 300, B=600, L=20, seed=87)
    _check(cfg, batch, S=16, C=16)


def test_hot_runs_above_a_tie():
    """200 runs of 50 lookups are hot; 100 tied runs of 40 are not."""
    cfg, batch = _tied_batch([50] * 200 + [40] * 100, B=700, L=20, seed=89)
    _check(cfg, batch, S=16, C=16)


def test_gradient_far_above_its_column_scale():
    """One gradient 1e8 times its column's first tile: the column is rescaled."""
    batch = make_batch(LARGE, B=2048)
    cfg = batch.cfg
    grad = batch.grad.copy()
    grad[1500, 3 * cfg.D + 17] = 1.0e8   # far above the column's first tile (about 3)
    batch = dataclasses.replace(batch, grad=grad)
    _check(cfg, batch, label="large skewed, one gradient of 1e8")


def test_small_first_tiles_rescale_columns_and_slots():
    """Gradients and weights of the first 16 bags of every 512 scaled by 1e-6:
    each segment's first tile sets scales 2^20 too small, and the later
    tiles move every column's and most hot slots' scales (and their
    accumulated values)."""
    batch = make_batch(LARGE, B=2048)
    cfg = batch.cfg
    grad = batch.grad.copy()
    psw = batch.psw.copy()
    small = (np.arange(cfg.B) % 512) < 16
    grad[small] *= np.float32(1e-6)
    for t in range(cfg.T):
        for b in np.nonzero(small)[0]:
            i = t * cfg.B + b
            psw[batch.offsets[i]:batch.offsets[i + 1]] *= np.float32(1e-6)
    batch = dataclasses.replace(batch, grad=grad, psw=psw)
    _check(cfg, batch, label="large skewed, small first tiles")


def test_bags_longer_than_staged():
    """Bags of 150 to 250 lookups: most of each bag's lookups are loaded in
    the build, and its H column is cleared whole afterwards."""
    cfg = Config("hot_long_bags", T=2, B=256, D=128, rows=(300, 300), dtype="bf16",
                 bag=("uniform", 150, 250), index=("zipf", 1.1), weighted=True,
                 preprocess_in_forward=True, seed=91)
    _check(cfg, make_batch(cfg), S=16, C=64)


def test_hot_rows_near_the_packed_hash_limit():
    """A table of 2^24 - 2 rows (its hot rows' packed entries row << 8 | slot
    reach the sign bit) beside a small one: the contraction runs."""
    cfg = Config("hot_rows_2p24m2", T=2, B=4096, D=32, rows=((1 << 24) - 2, 3000), dtype="bf16",
                 bag=("poisson", 20.0), index=("zipf", 1.2), weighted=True,
                 preprocess_in_forward=True, seed=97)
    batch = make_batch(cfg)
    pre = _check(cfg, batch, S=32, C=64)
    keys = pre["run_keys"].astype(np.int64)
    sl = np.diff(pre["run_offsets"].astype(np.int64))
    long_t0 = keys[(sl >= 32) & (keys < cfg.rows[0])]
    assert (long_t0 >= (1 << 23)).any(), "no long run of table 0 above 2^23"
    assert long_t0.size <= 256  # every one of them hot


def test_table_too_large_for_the_packed_hash_falls_back():
    """A table of 2^24 - 1 rows: the flag is ignored and the chunk path takes
    every long run, with the same result."""
    cfg = Config("hot_rows_2p24m1", T=2, B=4096, D=32, rows=((1 << 24) - 1, 3000), dtype="bf16",
                 bag=("poisson", 20.0), index=("zipf", 1.2), weighted=True,
                 preprocess_in_forward=True, seed=98)
    _check(cfg, make_batch(cfg), S=32, C=64, hot=False)
