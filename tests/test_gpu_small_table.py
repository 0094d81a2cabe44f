"""GPU parity of the small-table histogram path (E <= 64, 64 <= D <= 128,
L >= 64, f16, unweighted): per-bag counts bit-exact against the oracle's
histogram; outputs and updated rows against the oracle's plain definition."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import (TOL, assert_rows_match, assert_untouched_unchanged, fresh_params,
                              host_rows, oracle_all, rel_err, run_library)
from workloads import WORKLOADS, TINY, DEMO3, MEDIUM, LARGE, SMALL_TABLE, Batch, Config, make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401


def _check(cfg, batch, meta_in_forward=True, backward_meta=True, expect_saturated=False,
           expect_wide=False):
    print(f"\n[small-table] T={cfg.T} B={cfg.B} D={cfg.D} E={max(cfg.rows)} N={batch.indices.size} "
          f"meta_fwd={meta_in_forward} meta_bwd={backward_meta}", flush=True)
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W0, m0, uk)
    r = run_library(cfg, batch, W, m, meta_in_forward=meta_in_forward, backward_meta=backward_meta)
    assert r["path"] == 1
    pre, out, bw = oracle_all(cfg, batch, Wrows, mrows, uk)
    err = rel_err(r["out"].cpu().numpy(), out)
    assert err <= TOL[cfg.dtype], f"forward rel err {err:.3g}"
    H = oracle.histogram(cfg.T, cfg.B, 64, cfg.rows, batch.indices, batch.offsets)
    hist = r["meta"]["hist"].cpu().numpy().reshape(cfg.T, cfg.B, 64)
    np.testing.assert_array_equal(hist, np.minimum(H, 255))
    assert int(r["meta"]["counts"][4]) == int(expect_saturated)
    assert int(r["meta"]["counts"][5]) == int(expect_wide)
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"], "small-table")
    assert_untouched_unchanged(W0, W, m0, m, uk)
    return r


def _cfg(T, B, D, E, L, seed):
    return Config("small", T=T, B=B, D=D, rows=(E,) * T if isinstance(E, int) else tuple(E),
                  dtype="f16", bag=("fixed", L), index=("uniform",), weighted=False,
                  preprocess_in_forward=False, seed=seed)


def test_small_table_reduced_batch():
    cfg = SMALL_TABLE
    batch = make_batch(cfg, B=512)
    _check(batch.cfg, batch)


def test_forward_without_metadata_then_preprocess():
    """Forward given no metadata keeps its counts in the workspace; the
    metadata then comes from tbe_preprocess."""
    cfg = SMALL_TABLE
    batch = make_batch(cfg, B=700)
    _check(batch.cfg, batch, meta_in_forward=False)


def test_backward_without_saved_counts():
    cfg = SMALL_TABLE
    batch = make_batch(cfg, B=300)
    _check(batch.cfg, batch, meta_in_forward=True, backward_meta=False)


@pytest.mark.parametrize("D,E", [(64, 64), (96, 40), (128, 1), (100, 64)])
def test_shapes(D, E):
    cfg = _cfg(3, 200, D, E, 70, seed=D + E)
    batch = make_batch(cfg)
    _check(cfg, batch)


def _saturated_batch(long_len):
    rng = np.random.default_rng(7)
    T, B, D, E = 2, 96, 128, 64
    lengths = np.full(T * B, 80)
    lengths[5] = 300
    lengths[B + 7] = long_len
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    idx = rng.integers(0, E, size=offsets[-1]).astype(np.int32)
    idx[offsets[5]:offsets[6]] = 3
    idx[offsets[B + 7]:offsets[B + 8]] = 9
    cfg = _cfg(T, B, D, E, 80, seed=11)
    grad = rng.standard_normal((B, T * D)).astype(np.float32)
    return cfg, Batch(cfg=cfg, indices=idx, offsets=offsets, psw=None, grad=grad)


@pytest.mark.parametrize("meta_in_forward", [True, False])
def test_saturated_counts_are_recounted(meta_in_forward):
    """Bags with more than 255 lookups of one row (but at most 2048): the saved
    uint8 counts saturate, the flag is raised, and both directions recount
    from indices and still contract on the matrix cores."""
    cfg, batch = _saturated_batch(2048)
    _check(cfg, batch, meta_in_forward=meta_in_forward, expect_saturated=True)


@pytest.mark.parametrize("meta_in_forward", [True, False])
def test_counts_beyond_f16_exact_integers(meta_in_forward):
    """A bag with 2500 lookups of one row: counts above 2048 are not exact in
    f16, so both directions fall back to f32 arithmetic."""
    cfg, batch = _saturated_batch(2500)
    _check(cfg, batch, meta_in_forward=meta_in_forward, expect_saturated=True, expect_wide=True)


@pytest.mark.parametrize("meta_in_forward", [True, False])
def test_fused_check_counts_bad_indices_as_row_zero(meta_in_forward):
    """TBE_FLAG_CHECK on the small-table path: indices outside the 64 rows
    count as row 0 in both directions and set the error word."""
    from dataclasses import replace
    import bwd_tbe_pooled_amd as tbe
    batch = make_batch(SMALL_TABLE, B=256)
    cfg = batch.cfg
    rng = np.random.default_rng(5)
    pos = rng.choice(batch.indices.size, size=40, replace=False)
    bad = batch.indices.copy()
    bad[pos] = np.array([64, 65, 1000, -1, -64], dtype=np.int32)[pos % 5]
    fixed = batch.indices.copy()
    fixed[pos] = 0
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, fixed, batch.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W0, m0, uk)
    r = run_library(cfg, replace(batch, indices=bad), W, m, meta_in_forward=meta_in_forward,
                    flags=tbe.TBE_FLAG_CHECK, error_flags=err)
    assert int(err.item()) == tbe.TBE_ERROR_INDEX
    assert r["path"] == 1
    fb = replace(batch, indices=fixed)
    pre, out, bw = oracle_all(cfg, fb, Wrows, mrows, uk)
    assert rel_err(r["out"].cpu().numpy(), out) <= TOL[cfg.dtype]
    H = oracle.histogram(cfg.T, cfg.B, 64, cfg.rows, fixed, batch.offsets)
    np.testing.assert_array_equal(r["meta"]["hist"].cpu().numpy().reshape(cfg.T, cfg.B, 64),
                                  np.minimum(H, 255))
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"], "small checked")
    assert_untouched_unchanged(W0, W, m0, m, uk)
