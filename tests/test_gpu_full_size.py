"""Parity at the full sizes of the two large workloads, in the launch
configuration the benchmark times: T=32, E=2M, D=128 bf16, B=131072 weighted
with preprocessing in the forward (about 84M lookups); and the small-table
workload T=64, E=64, D=128 f16, B=32768, L=64 (134M lookups).

The large workload is also run with uniform rows (the same shapes, no
reuse, almost every run short).

The oracle cannot redo 84M lookups in seconds, so:
- the sort / RLE / routing metadata is checked by properties that define the
  stable sort uniquely (permutation; keys non-decreasing; equal keys in
  increasing position), exact RLE of the sorted keys, and the oracle's routing
  of the GPU's run lengths compared element by element;
- the forward is checked on 50,000 random bags spread over all tables;
- the backward is checked on every long run (segment length >= 256: the
  hot rows' contraction where the benchmark takes it, the chunk path, its
  per-XCD schedule and work queue, and the apply) and on
  short runs sampled evenly from each segment-length band (1, 2-4, 5-255),
  each row with every one of its lookups, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import (TOL, assert_rows_match, assert_untouched_unchanged, fresh_params,
                              host_rows, meta_host, rel_err, run_library)
from workloads import WORKLOADS, TINY, DEMO3, MEDIUM, LARGE, SMALL_TABLE, make_batch

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401


def _mask(n, members):
    mk = np.zeros(n, dtype=bool)
    mk[members] = True
    return mk


def _sampled_backward(cfg, batch, keys, bags, W, m, Wrows_all, mrows_all, uk, sample_keys,
                      label="sampled rows"):
    sel = _mask(cfg.sum_rows, sample_keys)[keys]
    pos = np.nonzero(sel)[0]
    sk = keys[pos]
    order = np.argsort(sk, kind="stable")          # stable: positions stay ascending
    pos = pos[order]
    sub_keys = keys[pos]
    sub_bags = bags[pos]
    sub_psw = None if batch.psw is None else batch.psw[pos]
    r = oracle.rle(sub_keys, np.arange(pos.size, dtype=np.int32), sub_bags, sub_psw)
    del sel, sk, order, sub_keys, sub_bags, sub_psw
    at = np.searchsorted(uk, r["run_keys"])
    bw = oracle.backward_adagrad(cfg.T, cfg.B, cfg.D, cfg.dtype, r["run_keys"], r["run_offsets"],
                                 r["sorted_bag"], r["sorted_psw"], batch.grad, Wrows_all[at],
                                 mrows_all[at], cfg.lr, cfg.eps, wkeys=r["run_keys"])
    err, ulps = assert_rows_match(cfg, W, m, r["run_keys"], bw["w_new"], bw["m_new"], label)
    print(f"[full] {label}: {r['run_keys'].size} rows, {pos.size} lookups, rel err {err:.2e}, "
          f"max {ulps} ulp", flush=True)
    return r["run_keys"].size, pos.size


def _backward_sample(counts, uk, rng, per_band=3000):
    """Every key of a long run (segment length >= 256) and up to `per_band`
    keys from each short band: 1, 2-4 and 5-255 lookups."""
    long_keys = uk[counts >= 256]
    bands = {}
    for name, lo, hi in (("SL 1", 1, 1), ("SL 2-4", 2, 4), ("SL 5-255", 5, 255)):
        cand = uk[(counts >= lo) & (counts <= hi)]
        bands[name] = (rng.choice(cand, min(per_band, cand.size), replace=False)
                       if cand.size else cand)
    return long_keys, bands


@pytest.mark.parametrize("rows,hot", [("zipf", True), ("zipf", False), ("uniform", True)],
                         ids=["zipf_hot_backward", "zipf_chunks_only", "uniform"])
def test_large_workload_full_size(rows, hot):
    """The benchmark's skewed batch (with the hot rows' backward on the
    matrix cores, as the benchmark runs it, and with every long run on the
    chunk path, the library's default), and the same shapes with uniform
    rows: 46.7M short runs, more than one round of the short-run kernel's
    grid (65536 workgroups of four waves, 64 runs each), so its waves
    stride."""
    import dataclasses
    import bwd_tbe_pooled_amd as tbe
    cfg = LARGE if rows == "zipf" else dataclasses.replace(LARGE, index=("uniform",))
    print(f"\n[full] generating the T=32 B=131072 workload, {rows} rows", flush=True)
    batch = make_batch(cfg)
    keys, bags = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    counts_all = np.bincount(keys, minlength=cfg.sum_rows)
    uk = np.nonzero(counts_all)[0].astype(np.int32)
    counts = counts_all[uk]
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    rng = np.random.default_rng(123)
    long_keys, bands = _backward_sample(counts, uk, rng)
    sample_keys = np.unique(np.concatenate([long_keys, *bands.values()])).astype(np.int32)
    sample_bags = rng.choice(cfg.T * cfg.B, 50_000, replace=False).astype(np.int32)
    assert np.unique(sample_bags // cfg.B).size == cfg.T
    need = np.unique(np.concatenate([sample_keys, keys[_mask(cfg.T * cfg.B, sample_bags)[bags]]]))
    Wrows, mrows = host_rows(W0, m0, need)
    print(f"[full] running the library, hot rows' backward {'on' if hot else 'off'}", flush=True)
    timer = tbe.Timer(4)
    r = run_library(cfg, batch, W, m, meta_in_forward=True, backward_meta=True, with_pos=False,
                    flags=tbe.TBE_FLAG_HOT_BACKWARD if hot else 0, timer=timer)
    if hot and rows == "zipf":
        assert timer.read()["bwd_hot"][1] == 1, "the hot rows' contraction did not run"

    # forward on sampled bags
    ob = oracle.forward_bags(cfg.D, cfg.dtype, batch.offsets, keys, batch.psw, Wrows, sample_bags,
                             wkeys=need)
    t, b = sample_bags // cfg.B, sample_bags % cfg.B
    out = r["out"].view(cfg.B, cfg.T, cfg.D)
    got = out[torch.from_numpy(b.astype(np.int64)).cuda(),
              torch.from_numpy(t.astype(np.int64)).cuda()].cpu().numpy()
    err = rel_err(got, ob)
    assert err <= TOL[cfg.dtype], f"forward rel err {err:.3g}"
    print(f"[full] forward: {sample_bags.size} bags of {cfg.T} tables, rel err {err:.2e}",
          flush=True)

    # metadata by defining properties and the oracle's routing
    print("[full] checking metadata", flush=True)
    h = meta_host(r["meta"], 0)
    N = keys.size
    assert h["sorted_pos"] is None          # the benchmark's configuration: no positions
    sp = np.argsort(keys, kind="stable")    # the stable order, by numpy's own sort
    ks = keys[sp]
    d = np.diff(ks)
    np.testing.assert_array_equal(h["sorted_bag"], bags[sp])
    np.testing.assert_array_equal(h["sorted_psw"].view(np.uint32), batch.psw[sp].view(np.uint32))
    heads = np.concatenate([[0], np.nonzero(d)[0] + 1])
    np.testing.assert_array_equal(h["run_offsets"], np.concatenate([heads, [N]]))
    np.testing.assert_array_equal(h["run_keys"], ks[heads])
    np.testing.assert_array_equal(h["run_keys"], uk)
    route = oracle.route(h["run_offsets"], 256, 256)
    for name in ("short_runs", "long_runs", "long_chunk_begin", "chunk_run", "chunk_start"):
        np.testing.assert_array_equal(h[name], route[name], err_msg=name)
    print(f"[full] U={uk.size} long={route['long_runs'].size} chunks={route['chunk_run'].size}",
          flush=True)
    if rows == "uniform":
        assert route["short_runs"].size > 65536 * 4 * 64

    # backward: every long run, then each short band, then untouched rows
    if long_keys.size:
        n_rows, n_look = _sampled_backward(cfg, batch, keys, bags, W, m, Wrows, mrows, need,
                                           long_keys, "every long run")
        assert n_rows == route["long_runs"].size
        assert n_look == int(counts[counts >= 256].sum())
    for name, band_keys in bands.items():
        if band_keys.size:
            _sampled_backward(cfg, batch, keys, bags, W, m, Wrows, mrows, need, band_keys, name)
    assert_untouched_unchanged(W0, W, m0, m, uk)


def test_small_table_workload_full_size():
    cfg = SMALL_TABLE
    print("\n[full] generating the T=64 B=32768 small-table workload", flush=True)
    batch = make_batch(cfg)
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    allk = np.arange(cfg.sum_rows, dtype=np.int32)
    Wrows, mrows = host_rows(W0, m0, allk)
    r = run_library(cfg, batch, W, m, meta_in_forward=True, backward_meta=True)
    assert r["path"] == 1
    rng = np.random.default_rng(5)
    sample_bags = rng.choice(cfg.T * cfg.B, 2000, replace=False).astype(np.int32)
    keys, bags = oracle.linearize(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets)
    ob = oracle.forward_bags(cfg.D, cfg.dtype, batch.offsets, keys, None, Wrows, sample_bags,
                             wkeys=allk)
    t, b = sample_bags // cfg.B, sample_bags % cfg.B
    out = r["out"].view(cfg.B, cfg.T, cfg.D)
    got = out[torch.from_numpy(b.astype(np.int64)).cuda(),
              torch.from_numpy(t.astype(np.int64)).cuda()].cpu().numpy()
    assert rel_err(got, ob) <= TOL[cfg.dtype]
    hist = r["meta"]["hist"].cpu().numpy().reshape(cfg.T * cfg.B, 64)
    for i in sample_bags[:500]:
        ref = np.bincount(batch.indices[batch.offsets[i]:batch.offsets[i + 1]], minlength=64)
        np.testing.assert_array_equal(hist[i], ref)
    assert int(r["meta"]["counts"][4]) == 0
    sample_keys = np.sort(rng.choice(cfg.sum_rows, 48, replace=False)).astype(np.int32)
    _sampled_backward(cfg, batch, keys, bags, W, m, Wrows, mrows, allk, sample_keys)
    assert_untouched_unchanged(W0, W, m0, m, allk)
