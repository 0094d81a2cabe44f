"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs. Metadata must match bit for bit; pooled outputs and
updated weights within the dtype's tolerance (1e-5 f32, 2e-3 f16, 1e-2 bf16,
max relative error floored at the row rms); optimizer state within 1e-5;
untouched rows bitwise unchanged."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import (TOL, assert_meta_equal, assert_rows_match,
                              assert_untouched_unchanged, fresh_params, host_rows,
                              make_desc, meta_host, oracle_all, rel_err, run_library)
from tests.helpers import TOL as _TOL  # noqa: F401
from workloads import WORKLOADS, TINY, DEMO3, MEDIUM, LARGE, SMALL_TABLE, Config, make_batch

pytestmark = pytest.mark.gpu

FUSED_LONG = 0x8  # TBE_FLAG_FUSED_LONG: long runs reduced and applied in the chunk kernel


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401  (fails loudly if the library is missing)


def _full_check(cfg, batch, *, meta_in_forward, backward_meta=True, S=0, C=0, m0="zeros",
                with_pos=True, flags=0):
    print(f"\n[parity] {cfg.name} T={cfg.T} B={cfg.B} D={cfg.D} {cfg.dtype} N={batch.indices.size} "
          f"S={S or 256} C={C or 256} meta_fwd={meta_in_forward} meta_bwd={backward_meta} "
          f"flags={flags:#x}", flush=True)
    W, m = fresh_params(cfg, m0)
    W0, m0t = W.clone(), m.clone()
    keys_all, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    uk = np.unique(keys_all)
    Wrows, mrows = host_rows(W0, m0t, uk)
    r = run_library(cfg, batch, W, m, meta_in_forward=meta_in_forward,
                    backward_meta=backward_meta, S=S, C=C, with_pos=with_pos, flags=flags)
    pre, out, bw = oracle_all(cfg, batch, Wrows, mrows, uk, S or 256, C or 256)
    err = rel_err(r["out"].cpu().numpy(), out)
    assert err <= TOL[cfg.dtype], f"forward rel err {err:.3g}"
    if r["path"] == 0:
        assert_meta_equal(meta_host(r["meta"], 0), pre)
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"], cfg.name)
    assert_untouched_unchanged(W0, W, m0t, m, uk)
    return r, pre


@pytest.mark.parametrize("name", ["tiny_t2_e1k_d16_f32", "demo3_d16_f32_b4k",
                                  "t16_e1m_d128_f16_b16k"])
def test_generic_workload_full(name):
    cfg = WORKLOADS[name]
    batch = make_batch(cfg)
    _full_check(cfg, batch, meta_in_forward=False, backward_meta=False)


def test_tiny_metadata_reused_from_preprocess():
    cfg = TINY
    _full_check(cfg, make_batch(cfg), meta_in_forward=False, backward_meta=True)


@pytest.mark.parametrize("flags", [0, FUSED_LONG], ids=["two_launch", "fused_long"])
def test_large_skewed_reduced_batch_full_compare(flags):
    cfg = LARGE
    batch = make_batch(cfg, B=2048)
    _full_check(batch.cfg, batch, meta_in_forward=True, backward_meta=True, flags=flags)


@pytest.mark.parametrize("T", [5, 13])
@pytest.mark.parametrize("flags", [0, FUSED_LONG], ids=["two_launch", "fused_long"])
def test_uneven_table_blocks_with_many_chunks(T, flags):
    """T not a multiple of the 8 XCDs: blocks of one or two tables, table
    pairs that hold one table; small S and C put most lookups on the chunked
    path, so every chunk of every per-XCD list must be served exactly once."""
    import dataclasses
    cfg = dataclasses.replace(LARGE, name=f"skewed_t{T}_e50k", T=T, rows=(50_000,) * T)
    batch = make_batch(cfg, B=1024)
    _full_check(batch.cfg, batch, meta_in_forward=True, S=16, C=8, flags=flags)


@pytest.mark.parametrize("name", ["demo3_d16_f32_b4k", "t16_e1m_d128_f16_b16k"])
def test_metadata_without_positions(name):
    """sorted_pos left NULL: the sort carries only bags and weights, which must
    still match the oracle's stable order bit for bit."""
    cfg = WORKLOADS[name]
    batch = make_batch(cfg, B=2048)
    _full_check(batch.cfg, batch, meta_in_forward=True, with_pos=False)


def test_large_skewed_reduced_batch_without_positions():
    cfg = LARGE
    batch = make_batch(cfg, B=1024)
    _full_check(batch.cfg, batch, meta_in_forward=True, with_pos=False)


@pytest.mark.parametrize("flags", [0, FUSED_LONG], ids=["two_launch", "fused_long"])
def test_demo3_fp64_partials_with_small_chunks(flags):
    """f32 weights accumulate and keep chunk partials in f64; small S/C put
    many runs on the chunked path."""
    cfg = DEMO3
    batch = make_batch(cfg, B=1024)
    _full_check(batch.cfg, batch, meta_in_forward=True, S=4, C=3, flags=flags)


def test_nonzero_initial_state():
    cfg = MEDIUM
    batch = make_batch(cfg, B=256)
    _full_check(batch.cfg, batch, meta_in_forward=True, m0="uniform")


# --- edge cases ---------------------------------------------------------------

def _custom(T, B, D, rows, dtype, lengths, indices, psw=None, seed=0):
    rng = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cfg = Config("edge", T=T, B=B, D=D, rows=tuple(rows), dtype=dtype, bag=("fixed", 0),
                 index=("uniform",), weighted=psw is not None, preprocess_in_forward=True,
                 seed=seed)
    from workloads import Batch
    grad = rng.standard_normal((B, T * D)).astype(np.float32)
    return cfg, Batch(cfg=cfg, indices=np.asarray(indices, dtype=np.int32), offsets=offsets,
                      psw=None if psw is None else np.asarray(psw, dtype=np.float32), grad=grad)


@pytest.mark.parametrize("flags", [0, FUSED_LONG], ids=["two_launch", "fused_long"])
@pytest.mark.parametrize("sl", [255, 256, 257, 511, 512, 513])
def test_segment_lengths_around_the_threshold(sl, flags):
    """One hot row hit exactly sl times, spread over bags, among cold rows."""
    rng = np.random.default_rng(sl)
    T, B, D = 2, 600, 16
    rows = [5000, 3000]
    lengths = rng.integers(1, 4, size=T * B)
    N = int(lengths.sum())
    idx = rng.integers(0, 3000, size=N)
    hot = rng.choice(int(lengths[:B].sum()), size=sl, replace=False)
    idx[hot] = 4242
    cfg, batch = _custom(T, B, D, rows, "f16" if sl % 2 else "bf16", lengths, idx,
                         psw=rng.random(N), seed=sl)
    r, pre = _full_check(cfg, batch, meta_in_forward=True, flags=flags)
    u = int(np.searchsorted(pre["run_keys"], 4242))
    assert pre["run_keys"][u] == 4242 and np.diff(pre["run_offsets"])[u] == sl
    assert (u in pre["long_runs"]) == (sl >= 256)


def test_every_lookup_on_one_row():
    T, B, D = 1, 4000, 128
    lengths = np.full(B, 7)
    cfg, batch = _custom(T, B, D, [100], "bf16", lengths, np.full(lengths.sum(), 17),
                         psw=np.random.default_rng(1).random(lengths.sum()))
    r, pre = _full_check(cfg, batch, meta_in_forward=True)
    assert pre["U"] == 1 and pre["chunk_run"].size == -(-lengths.sum() // 256)


def test_empty_bags_and_all_empty_batch():
    rng = np.random.default_rng(3)
    T, B, D = 3, 500, 3
    lengths = rng.integers(0, 5, size=T * B)
    lengths[rng.random(T * B) < 0.6] = 0
    idx = rng.integers(0, 40, size=lengths.sum())
    cfg, batch = _custom(T, B, D, [40, 41, 42], "f32", lengths, idx)
    r, _ = _full_check(cfg, batch, meta_in_forward=True)
    out = r["out"].cpu().numpy().reshape(B, T, D)
    L = lengths.reshape(T, B)
    for t in range(T):
        assert not out[L[t] == 0, t].any()
    cfg0, batch0 = _custom(2, 64, 16, [10, 10], "f32", np.zeros(128, dtype=np.int64), [])
    r0, pre0 = _full_check(cfg0, batch0, meta_in_forward=True)
    assert pre0["U"] == 0 and not r0["out"].any()


def test_zero_bags():
    """B = 0: no bags, no lookups, an empty output; every call (int32 and
    int64, metadata and not) succeeds and leaves the weights alone."""
    import bwd_tbe_pooled_amd as tbe
    from tests.gpu_common import make_desc
    cfg = Config("zero_bags", T=3, B=0, D=16, rows=(10, 20, 30), dtype="f32", bag=("fixed", 0),
                 index=("uniform",), weighted=False, preprocess_in_forward=True, seed=0)
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    idx = torch.zeros(0, dtype=torch.int32, device="cuda")
    off = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((0, cfg.T * cfg.D), dtype=torch.float32, device="cuda")
    grad = torch.empty((0, cfg.T * cfg.D), dtype=torch.float32, device="cuda")
    desc = make_desc(cfg)
    meta = tbe.Meta(desc, 0, False)
    tbe.tbe_forward(desc, W, idx, off, None, out, meta,
                    tbe.workspace(desc, 0, False, tbe.TBE_OP_FORWARD_PREPROCESS))
    tbe.tbe_backward_adagrad(desc, W, m, grad, idx, off, None, meta, cfg.lr, cfg.eps,
                             tbe.workspace(desc, 0, False, tbe.TBE_OP_BACKWARD))
    tbe.tbe_backward_adagrad(desc, W, m, grad, idx, off, None, None, cfg.lr, cfg.eps,
                             tbe.workspace(desc, 0, False, tbe.TBE_OP_BACKWARD_SELF))
    tbe.tbe_forward_i64(desc, W, idx.long(), off.long(), None, out,
                        tbe.workspace_i64(desc, 0, False, tbe.TBE_OP_FORWARD))
    tbe.tbe_backward_adagrad_i64(desc, W, m, grad, idx.long(), off.long(), None, cfg.lr, cfg.eps,
                                 tbe.workspace_i64(desc, 0, False, tbe.TBE_OP_BACKWARD_SELF))
    torch.cuda.synchronize()
    assert int(meta["counts"][0].item()) == 0
    assert torch.equal(W, W0) and torch.equal(m, m0)


@pytest.mark.parametrize("flags", [0, FUSED_LONG], ids=["two_launch", "fused_long"])
@pytest.mark.parametrize("D", [1, 3, 24, 256, 1000])
def test_odd_dimensions(D, flags):
    rng = np.random.default_rng(D)
    T, B = 2, 300
    lengths = rng.poisson(6, size=T * B)
    idx = rng.integers(0, 30, size=lengths.sum())
    cfg, batch = _custom(T, B, D, [30, 50], "f16" if D % 2 == 0 else "f32", lengths, idx,
                         psw=rng.random(lengths.sum()), seed=D)
    _full_check(cfg, batch, meta_in_forward=True, S=8, C=5, flags=flags)


def test_unit_weights_equal_unweighted_bitwise():
    cfg = MEDIUM
    batch = make_batch(cfg, B=512)
    outs = []
    for psw in (None, np.ones(batch.indices.size, dtype=np.float32)):
        b = make_batch(cfg, B=512)
        b.psw = psw
        W, m = fresh_params(batch.cfg)
        r = run_library(batch.cfg, b, W, m, meta_in_forward=True)
        outs.append((r["out"].clone(), W.clone(), m.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.float16 else a,
                           b.view(torch.int16) if b.dtype == torch.float16 else b)


def test_runs_are_deterministic():
    cfg = LARGE
    batch = make_batch(cfg, B=4096)
    res = []
    for _ in range(2):
        W, m = fresh_params(batch.cfg)
        r = run_library(batch.cfg, batch, W, m, meta_in_forward=True)
        res.append((r["out"], W.view(torch.int16), m))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


def test_validate_flag_reports_bad_input_before_other_work():
    import bwd_tbe_pooled_amd as tbe
    cfg = TINY
    batch = make_batch(cfg)
    desc = make_desc(cfg, flags=tbe.TBE_FLAG_VALIDATE)
    W, m = fresh_params(cfg)
    out = torch.zeros((cfg.B, cfg.T * cfg.D), device="cuda")
    ws = tbe.workspace(desc, batch.indices.size, False, tbe.TBE_OP_FORWARD)
    off = torch.from_numpy(batch.offsets).cuda()
    good = torch.from_numpy(batch.indices).cuda()
    tbe.tbe_forward(desc, W, good, off, None, out, None, ws)      # valid input passes
    bad = good.clone()
    bad[5] = cfg.rows[0]                                            # one past the table
    out2 = torch.zeros_like(out)
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_forward(desc, W, bad, off, None, out2, None, ws)
    assert e.value.status == tbe.TBE_ERR_INDEX_RANGE
    assert not out2.any()                                           # nothing else ran
    bad_off = off.clone()
    bad_off[3] = bad_off[4] + 1                                     # decreasing offsets
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_forward(desc, W, good, bad_off, None, out2, None, ws)
    assert e.value.status == tbe.TBE_ERR_INDEX_RANGE


def test_stage_timer_counts_each_stage():
    import bwd_tbe_pooled_amd as tbe
    cfg = MEDIUM
    batch = make_batch(cfg, B=1024)
    timer = tbe.Timer(8)
    desc = make_desc(batch.cfg, timer=timer)
    W, m = fresh_params(batch.cfg)
    from tests.gpu_common import device_batch
    dev = device_batch(batch)
    N = batch.indices.size
    meta = tbe.Meta(desc, N, False)
    out = torch.empty((batch.cfg.B, cfg.T * cfg.D), device="cuda")
    ws = tbe.workspace(desc, N, False, tbe.TBE_OP_FORWARD_PREPROCESS)
    tbe.tbe_forward(desc, W, dev["indices"], dev["offsets"], None, out, meta, ws)
    wsb = tbe.workspace(desc, N, False, tbe.TBE_OP_BACKWARD)
    tbe.tbe_backward_adagrad(desc, W, m, dev["grad"], dev["indices"], dev["offsets"], None, meta,
                             0.01, 1e-8, wsb)
    t = timer.read()
    for st in ("fwd_pool", "linearize", "sort", "rle_route", "bwd_short", "long_schedule",
               "bwd_long", "bwd_apply"):
        assert t[st][1] == 1 and t[st][0] > 0, st
    for st in ("small_count", "small_fwd", "small_bwd", "small_apply", "validate"):
        assert t[st][1] == 0, st


# --- bounds check fused into the kernels (TBE_FLAG_CHECK) -------------------

def _plant_bad_indices(batch, seed, count=24):
    """Copy of the batch with `count` indices moved outside their tables, and
    the batch the oracle should see: those lookups read as row 0."""
    from dataclasses import replace
    rng = np.random.default_rng(seed)
    N = batch.indices.size
    pos = rng.choice(N, size=min(count, N), replace=False)
    bad = batch.indices.copy()
    big = np.array([10 ** 9, 2 ** 31 - 1, -1, -7], dtype=np.int64)
    bad[pos] = np.where(rng.random(pos.size) < 0.5,
                        max(batch.cfg.rows) + rng.integers(0, 5, pos.size), big[pos % 4])
    fixed = batch.indices.copy()
    fixed[pos] = 0
    return replace(batch, indices=bad), replace(batch, indices=fixed)


@pytest.mark.parametrize("name,B,meta_fwd", [("t16_e1m_d128_f16_b16k", 512, True),
                                             ("t32_e2m_d128_bf16_b128k", 1024, True),
                                             ("t32_e2m_d128_bf16_b128k", 1024, False)])
def test_fused_check_reads_bad_indices_as_row_zero(name, B, meta_fwd):
    import bwd_tbe_pooled_amd as tbe
    batch = make_batch(WORKLOADS[name], B=B)
    cfg = batch.cfg
    bad, fixed = _plant_bad_indices(batch, seed=len(name) + B + int(meta_fwd))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    keys, _ = oracle.linearize(cfg.T, cfg.B, cfg.rows, fixed.indices, fixed.offsets)
    uk = np.unique(keys)
    Wrows, mrows = host_rows(W0, m0, uk)
    r = run_library(cfg, bad, W, m, meta_in_forward=meta_fwd, flags=tbe.TBE_FLAG_CHECK,
                    error_flags=err)
    assert int(err.item()) == tbe.TBE_ERROR_INDEX
    pre, out, bw = oracle_all(cfg, fixed, Wrows, mrows, uk, 256, 256)
    assert rel_err(r["out"].cpu().numpy(), out) <= TOL[cfg.dtype]
    assert_meta_equal(meta_host(r["meta"], 0), pre)
    assert_rows_match(cfg, W, m, pre["run_keys"], bw["w_new"], bw["m_new"], "checked")
    assert_untouched_unchanged(W0, W, m0, m, uk)


def test_fused_check_is_silent_and_bitwise_neutral_on_valid_input():
    import bwd_tbe_pooled_amd as tbe
    batch = make_batch(LARGE, B=1024)
    cfg = batch.cfg
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = []
    for flags in (0, tbe.TBE_FLAG_CHECK):
        W, m = fresh_params(cfg)
        r = run_library(cfg, batch, W, m, meta_in_forward=True, flags=flags, error_flags=err)
        res.append((r["out"], W.view(torch.int16), m))
    assert int(err.item()) == 0
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


def test_binding_rejects_mistyped_tensors():
    """int64 indices given to the int32 calls, strided outputs, wrong weight
    dtypes and wrong sizes are refused with a TypeError before any launch."""
    import bwd_tbe_pooled_amd as tbe
    cfg = TINY
    batch = make_batch(cfg)
    desc = make_desc(cfg)
    dev = "cuda"
    idx = torch.from_numpy(batch.indices).to(dev)
    off = torch.from_numpy(batch.offsets).to(dev)
    W, m = fresh_params(cfg)
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device=dev)
    ws = tbe.workspace(desc, idx.numel(), False, tbe.TBE_OP_FORWARD)
    bad = [
        dict(indices=idx.long()),                                   # int64 as int32
        dict(offsets=off.long()),
        dict(offsets=off[:-1]),                                     # T*B offsets, not T*B + 1
        dict(W=W.half()),                                           # weight dtype
        dict(out=torch.empty((cfg.T * cfg.D, cfg.B), device=dev).t()),  # strided view
        dict(out=torch.empty((cfg.B, cfg.T * cfg.D + 1), device=dev)),
    ]
    for b in bad:
        a = dict(W=W, indices=idx, offsets=off, out=out)
        a.update(b)
        with pytest.raises(TypeError):
            tbe.tbe_forward(desc, a["W"], a["indices"], a["offsets"], None, a["out"], None, ws)
    grad = torch.zeros((cfg.B, cfg.T * cfg.D), device=dev)
    with pytest.raises(TypeError):
        tbe.tbe_backward_adagrad(desc, W, m.double(), grad, idx, off, None, None, cfg.lr, cfg.eps,
                                 tbe.workspace(desc, idx.numel(), False, tbe.TBE_OP_BACKWARD_SELF))
