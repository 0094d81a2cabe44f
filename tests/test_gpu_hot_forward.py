"""The forward that runs after the transpose reads the hottest rows of each
table from LDS and the rest from global memory, and sums a bag's hot rows
before its cold ones. Its output is compared with the oracle on the whole
batch (as is the plain gather's, given no metadata, on the same inputs), and
the metadata it writes must equal that of tbe_preprocess, and the stage timer
must show that the hot rows were taken. Checked on weighted and unweighted
bf16 (rows held widened to f32 in LDS), bf16 rows of 96 (four idle lanes per
row slot), empty bags, unweighted f16 and f32 rows of 16, with more and with fewer long runs
than the hot rows a table holds (127 widened bf16 rows of 512 bytes at D = 128),
with bags longer than one staged window
of 128 lookups, and with the fused bounds check on planted bad indices (read
as row 0, as the oracle is told)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import device_batch, fresh_params, make_desc, meta_host, raw_bits, rel_err
from workloads import DEMO3, LARGE, MEDIUM, make_batch

# f32 sums of f16/bf16 rows, f64 sums of f32 rows, each rounded to f32 once
FWD_TOL = {"f32": 1e-6, "f16": 1e-5, "bf16": 1e-5}

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401


def _forward_pair(cfg, batch, flags=0, S=0, dev=None, oracle_indices=None):
    import bwd_tbe_pooled_amd as tbe
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    d1 = make_desc(cfg, S=S, flags=flags, error_flags=err1)
    d2 = make_desc(cfg, S=S, flags=flags, error_flags=err2)
    dev = dev or device_batch(batch)
    N = batch.indices.size
    weighted = batch.psw is not None
    W, _ = fresh_params(cfg)
    out_hot = torch.full((cfg.B, cfg.T * cfg.D), float("nan"), device="cuda")
    out_plain = torch.full((cfg.B, cfg.T * cfg.D), float("nan"), device="cuda")
    meta = tbe.Meta(d1, N, weighted)
    timer = tbe.Timer(4)
    d1.set_timer(timer)
    tbe.tbe_forward(d1, W, dev["indices"], dev["offsets"], dev["psw"], out_hot, meta,
                    tbe.workspace(d1, N, weighted, tbe.TBE_OP_FORWARD_PREPROCESS))
    d1.set_timer(None)
    tbe.tbe_forward(d2, W, dev["indices"], dev["offsets"], dev["psw"], out_plain, None,
                    tbe.workspace(d2, N, weighted, tbe.TBE_OP_FORWARD))
    meta2 = tbe.Meta(d2, N, weighted)
    tbe.tbe_preprocess(d2, dev["indices"], dev["offsets"], dev["psw"], meta2,
                       tbe.workspace(d2, N, weighted, tbe.TBE_OP_PREPROCESS))
    torch.cuda.synchronize()
    # the case is only a test of the forward after the transpose if it took the hot rows
    assert timer.read()["hot_plan"][1] == 1, "the forward after the transpose did not run"
    idx = batch.indices if oracle_indices is None else oracle_indices
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, idx, batch.offsets)
    need = np.unique(keys)
    Wrows = raw_bits(W.index_select(0, torch.from_numpy(need.astype(np.int64)).cuda()))
    ref = oracle.forward(cfg.T, cfg.B, cfg.D, cfg.dtype, batch.offsets, keys, batch.psw, Wrows,
                         wkeys=need)
    e_hot = rel_err(out_hot.cpu().numpy(), ref)
    e_plain = rel_err(out_plain.cpu().numpy(), ref)
    print(f"\n[hot] {cfg.name} B={cfg.B}: rel err {e_hot:.2e} (plain gather {e_plain:.2e})",
          flush=True)
    assert e_hot <= FWD_TOL[cfg.dtype] and e_plain <= FWD_TOL[cfg.dtype]
    h1, h2 = meta_host(meta, 0), meta_host(meta2, 0)
    np.testing.assert_array_equal(h1["counts"][:4], h2["counts"][:4])   # [4..7] unused here
    for k in h1:
        if k != "counts" and h1[k] is not None:
            np.testing.assert_array_equal(h1[k], h2[k], err_msg=k)
    return int(h1["counts"][2]), int(err1.item()), int(err2.item())


def _cfg(name, **kw):
    from workloads import Config
    base = dict(T=8, B=8192, D=128, rows=(3000,) * 8, dtype="bf16", bag=("poisson", 20.0),
                index=("zipf", 1.05), weighted=True, preprocess_in_forward=True, seed=79)
    base.update(kw)
    return Config(name, **base)


@pytest.mark.parametrize("name,cfg,B", [
    ("bf16_weighted", LARGE, 2048),        # 13-15 long runs per table: fewer than 127
    ("bf16_unweighted", dataclasses.replace(LARGE, weighted=False), 2048),
    # 12 of a slot's 16 lanes hold the row; 169 widened rows per table
    ("bf16_d96", _cfg("hot_d96", D=96), 8192),
    # about 5% of the bags are empty
    ("bf16_empty_bags", _cfg("hot_empty", rows=(2000,) * 8, bag=("poisson", 3.0),
                             index=("zipf", 1.1)), 8192),
    ("f16", MEDIUM, 16384),
    ("f32_d16", dataclasses.replace(DEMO3, B=32768), 32768),
])
def test_forward_after_transpose_equals_plain_gather(name, cfg, B):
    batch = make_batch(cfg, B=B)
    n_long, _, _ = _forward_pair(batch.cfg, batch)
    print(f"[hot] {name}: {n_long} long runs", flush=True)
    assert n_long > 0


def test_forward_after_transpose_many_hot_rows():
    """More than 256 long runs per table (uniform rows over 600 per table,
    about 136 lookups each, with S = 16): the plan keeps the 255 longest
    (one LDS row of the 64 KB holds zeros)."""
    from workloads import Config
    cfg = Config("hot_many", T=64, B=4096, D=128, rows=(600,) * 64, dtype="bf16",
                 bag=("fixed", 20), index=("uniform",), weighted=True,
                 preprocess_in_forward=True, seed=71)
    batch = make_batch(cfg)
    n_long, _, _ = _forward_pair(cfg, batch, S=16)
    assert n_long >= 600 * 64 * 0.9


def test_forward_after_transpose_many_long_runs_per_table():
    """About 6000 long runs per table (uniform rows over 6000 per table, about
    27 lookups each, with S = 16): more runs than the plan holds in LDS, so it
    reads their lengths from the run list at every count."""
    from workloads import Config
    cfg = Config("hot_many_runs", T=8, B=8192, D=128, rows=(6000,) * 8, dtype="bf16",
                 bag=("fixed", 20), index=("uniform",), weighted=True,
                 preprocess_in_forward=True, seed=73)
    batch = make_batch(cfg)
    n_long, _, _ = _forward_pair(cfg, batch, S=16)
    assert n_long > 8 * 4096


def test_forward_after_transpose_with_fused_bounds_check():
    import bwd_tbe_pooled_amd as tbe
    batch = make_batch(LARGE, B=2048)
    cfg = batch.cfg
    idx = batch.indices.copy()
    rng = np.random.default_rng(3)
    at = rng.choice(idx.size, 50, replace=False)
    idx[at[:25]] = cfg.rows[0] + 5      # beyond the table
    idx[at[25:]] = -7
    batch = dataclasses.replace(batch, indices=idx)
    fixed = idx.copy()
    fixed[at] = 0
    _, e1, e2 = _forward_pair(cfg, batch, flags=tbe.TBE_FLAG_CHECK, oracle_indices=fixed)
    assert e1 == tbe.TBE_ERROR_INDEX and e2 == tbe.TBE_ERROR_INDEX


def test_forward_after_transpose_long_bags():
    """Bags of 150-300 lookups: a group of bags spans several staged windows,
    and a bag's cold rows need several batches (8 tables of 8192 bags: enough
    workgroups for the forward after the transpose)."""
    from workloads import Config
    cfg = Config("hot_long_bags", T=8, B=8192, D=64, rows=(3000,) * 8, dtype="bf16",
                 bag=("uniform", 150, 300), index=("zipf", 1.05), weighted=True,
                 preprocess_in_forward=True, seed=73)
    batch = make_batch(cfg)
    n_long, _, _ = _forward_pair(cfg, batch)
    assert n_long > 0
