"""Upstream gradients at the edges of the arithmetic, through the C ABI
against the oracle:
- an infinite gradient row of bag (t, 0) must reach only the rows that bag
  looks up: every other row stays finite and matches the oracle (the
  backward's gather lanes past the end of a run load nothing);
- on the small-table path, the compensated f16 hi/lo split works on each
  gradient column scaled by a power of two: gradients far below 1 (which
  unscaled would fall into f16's subnormals and lose most of their bits) and
  far above f16's largest value match the oracle, and a tile far outside its
  column's scale is redone in f32 arithmetic."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import (TOL, assert_rows_match, fresh_params, host_rows, oracle_all,
                              rel_err, run_library)
from workloads import MEDIUM, SMALL_TABLE, make_batch, table_offsets

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401


@pytest.mark.parametrize("S,C", [(256, 256), (16, 8)])
def test_infinite_gradient_row_stays_in_its_own_rows(S, C):
    batch = make_batch(MEDIUM, B=2048)
    cfg = batch.cfg
    grad = batch.grad.copy()
    for t in range(cfg.T):
        grad[0, t * cfg.D:(t + 1) * cfg.D] = np.inf
    batch.grad = grad
    print(f"\n[edge] inf gradient rows of bag 0, S={S} C={C}", flush=True)
    toff = table_offsets(cfg.rows)
    hit = np.unique(np.concatenate([
        toff[t] + batch.indices[batch.offsets[t * cfg.B]:batch.offsets[t * cfg.B + 1]]
        for t in range(cfg.T)]))
    W, m = fresh_params(cfg)
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W, m, uk)
    r = run_library(cfg, batch, W, m, meta_in_forward=True, S=S, C=C)
    pre, _, bw = oracle_all(cfg, batch, Wrows, mrows, uk, S=S, C=C)
    counts = r["meta"]["counts"].cpu().numpy()
    assert int(counts[2]) > 0, "the batch must have long runs"
    inf_rows = np.isin(pre["run_keys"], hit)
    assert inf_rows.any() and not inf_rows.all()
    fin = ~inf_rows
    assert np.isfinite(bw["w_new"][fin]).all()
    assert_rows_match(cfg, W, m, pre["run_keys"][fin], bw["w_new"][fin], bw["m_new"][fin],
                      "rows bag 0 does not look up")
    kt = torch.from_numpy(pre["run_keys"][inf_rows].astype(np.int64)).cuda()
    assert not torch.isfinite(W.index_select(0, kt).float()).all(dim=1).any()


def test_small_table_gradients_beyond_f16_range():
    """Entries above 65504 in a few bags: the first tile's 1e5 sets its
    column's scale; 3e9 in a later tile is beyond that scale and its split is
    redone in f32."""
    batch = make_batch(SMALL_TABLE, B=1024)
    cfg = batch.cfg
    grad = batch.grad.copy()
    rng = np.random.default_rng(11)
    # a few entries beyond f16's largest finite value (65504), in some tables
    # and bags only, so that most splits stay on the matrix cores
    for b, col, v in [(3, 5, 1.0e5), (700, 40 * cfg.D + 17, -7.0e4), (1001, 9 * cfg.D, 65504.0),
                      (512, 63 * cfg.D + cfg.D - 1, 3.0e9)]:
        grad[b, col] = v
    batch.grad = grad
    print(f"\n[edge] small-table gradients up to 3e9", flush=True)
    W, m = fresh_params(cfg)
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W, m, uk)
    r = run_library(cfg, batch, W, m, meta_in_forward=True)
    assert r["path"] == 1
    pre, out, bw = oracle_all(cfg, batch, Wrows, mrows, uk)
    assert int(r["meta"]["counts"][5]) == 0      # counts are small: only the gradients are wide
    assert np.isfinite(bw["w_new"]).all()
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"], "small-table wide g")
    assert rel_err(r["out"].cpu().numpy(), out) <= TOL[cfg.dtype]


@pytest.mark.parametrize("scale", [1e-6, 1e-15, 1e12])
def test_small_table_gradient_magnitudes(scale):
    """The whole upstream gradient times `scale`. At 1e-6 an unscaled f16 split
    would keep about 15 bits of each gradient (f16's subnormals start at
    6e-5), enough to put the Adagrad state off by several 1e-5."""
    batch = make_batch(SMALL_TABLE, B=2048)
    cfg = batch.cfg
    batch.grad = (batch.grad.astype(np.float64) * scale).astype(np.float32)
    print(f"\n[edge] small-table gradients times {scale:g}", flush=True)
    W, m = fresh_params(cfg)
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W, m, uk)
    r = run_library(cfg, batch, W, m, meta_in_forward=True)
    assert r["path"] == 1
    pre, _, bw = oracle_all(cfg, batch, Wrows, mrows, uk)
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"],
                      f"small-table g x {scale:g}")


def test_small_table_gradient_magnitudes_per_bag():
    """Each bag's gradient row times 10^u, u uniform in [-6, 0]: one column
    mixes magnitudes six decades apart, within the split's scaled range."""
    batch = make_batch(SMALL_TABLE, B=2048)
    cfg = batch.cfg
    rng = np.random.default_rng(19)
    f = 10.0 ** rng.uniform(-6, 0, size=(cfg.B, 1))
    batch.grad = (batch.grad.astype(np.float64) * f).astype(np.float32)
    W, m = fresh_params(cfg)
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W, m, uk)
    r = run_library(cfg, batch, W, m, meta_in_forward=True)
    assert r["path"] == 1
    pre, _, bw = oracle_all(cfg, batch, Wrows, mrows, uk)
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"],
                      "small-table g per-bag magnitudes")
