"""int64 indices and offsets (page 1, checklist item 6) through the C ABI.

- Problems within the int32 limits: the int64 entry points must give the same
  bits as the int32 ones (forward; backward that preprocesses itself), which
  the parity tests compare with the oracle.
- Rows beyond 2^31 in total (three tables of 1.2e9, 1.0e9 and 0.5e9 rows):
  each table is compared with the oracle run on that table alone. Tables are
  independent in the method (every run belongs to one table), so this is the
  oracle's result for the whole call.
- Lookups beyond 2^31 (2.2e9): an index pattern whose lookups per row are
  known in closed form; sampled bags and rows against the oracle.
- Index values outside int32 are read as row 0 and flagged under the fused
  check, exactly like out-of-table int32 indices; the validation flag rejects
  them before any update; inconsistent table offsets are rejected."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import (assert_rows_match, device_batch, fresh_params, lib, make_desc,
                              rel_err, TOL)
from workloads import WORKLOADS, make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401  (fails loudly if the library is missing)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _step(cfg, dev, idx, off, wide, flags=0, err=None):
    """Forward (no metadata) and backward (preprocessing itself) through the
    int32 or the int64 entry points. Returns out, W, m."""
    tbe = lib()
    desc = make_desc(cfg, flags=flags, error_flags=err)
    N = idx.numel()
    weighted = dev["psw"] is not None
    W, m = fresh_params(cfg)
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device="cuda")
    if wide:
        ws = tbe.workspace_i64(desc, N, weighted, tbe.TBE_OP_FORWARD)
        tbe.tbe_forward_i64(desc, W, idx, off, dev["psw"], out, ws)
        del ws
        ws = tbe.workspace_i64(desc, N, weighted, tbe.TBE_OP_BACKWARD_SELF)
        tbe.tbe_backward_adagrad_i64(desc, W, m, dev["grad"], idx, off, dev["psw"], cfg.lr,
                                     cfg.eps, ws)
    else:
        ws = tbe.workspace(desc, N, weighted, tbe.TBE_OP_FORWARD)
        tbe.tbe_forward(desc, W, idx, off, dev["psw"], out, None, ws)
        del ws
        ws = tbe.workspace(desc, N, weighted, tbe.TBE_OP_BACKWARD_SELF)
        tbe.tbe_backward_adagrad(desc, W, m, dev["grad"], idx, off, dev["psw"], None, cfg.lr,
                                 cfg.eps, ws)
    torch.cuda.synchronize()
    return out, W, m


@pytest.mark.parametrize("name,B", [("demo3_d16_f32_b4k", None), ("t16_e1m_d128_f16_b16k", 2048),
                                    ("t32_e2m_d128_bf16_b128k", 1024),
                                    ("small_t64_e64_d128_f16_b32k", 512)])
def test_int64_entry_points_match_int32_bitwise(name, B):
    batch = make_batch(WORKLOADS[name], B=B)
    cfg = batch.cfg
    print(f"\n[int64] {cfg.name} T={cfg.T} B={cfg.B} N={batch.indices.size}", flush=True)
    dev = device_batch(batch)
    o32, W32, m32 = _step(cfg, dev, dev["indices"], dev["offsets"], wide=False)
    o64, W64, m64 = _step(cfg, dev, dev["indices"].long(), dev["offsets"].long(), wide=True)
    assert torch.equal(_bits(o32), _bits(o64)), "forward differs"
    assert torch.equal(_bits(W32), _bits(W64)), "weights differ"
    assert torch.equal(_bits(m32), _bits(m64)), "state differs"


def test_int64_values_outside_int32_are_flagged_and_read_as_row_zero():
    tbe = lib()
    batch = make_batch(WORKLOADS["t16_e1m_d128_f16_b16k"], B=512)
    cfg = batch.cfg
    dev = device_batch(batch)
    rng = np.random.default_rng(5)
    pos = torch.from_numpy(rng.choice(batch.indices.size, 40, replace=False)).cuda()
    wide = dev["indices"].long()
    wide[pos[:20]] = 2 ** 32 + 5          # would wrap to row 5 if cut to 32 bits
    wide[pos[20:30]] = -3
    wide[pos[30:]] = 2 ** 40
    narrow = dev["indices"].clone()
    narrow[pos] = -1                      # out of every table as int32
    e32 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e64 = torch.zeros(1, dtype=torch.int32, device="cuda")
    r32 = _step(cfg, dev, narrow, dev["offsets"], False, tbe.TBE_FLAG_CHECK, e32)
    r64 = _step(cfg, dev, wide, dev["offsets"].long(), True, tbe.TBE_FLAG_CHECK, e64)
    assert int(e32.item()) == tbe.TBE_ERROR_INDEX and int(e64.item()) == tbe.TBE_ERROR_INDEX
    for a, b in zip(r32, r64):
        assert torch.equal(_bits(a), _bits(b))


def test_int64_validation_and_offsets_checks():
    tbe = lib()
    batch = make_batch(WORKLOADS["demo3_d16_f32_b4k"], B=256)
    cfg = batch.cfg
    dev = device_batch(batch)
    N = batch.indices.size
    idx = dev["indices"].long()
    idx[N // 2] = 2 ** 33
    off = dev["offsets"].long()
    W, m = fresh_params(cfg)
    W0 = W.clone()
    desc = make_desc(cfg, flags=tbe.TBE_FLAG_VALIDATE)
    ws = tbe.workspace_i64(desc, N, False, tbe.TBE_OP_BACKWARD_SELF)
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_backward_adagrad_i64(desc, W, m, dev["grad"], idx, off, None, cfg.lr, cfg.eps, ws)
    assert e.value.status == tbe.TBE_ERR_INDEX_RANGE
    torch.cuda.synchronize()
    assert torch.equal(_bits(W), _bits(W0))
    # table boundaries that do not add up to N are refused before any work
    bad_off = off.clone()
    bad_off[-1] = N + 7
    plain = make_desc(cfg)
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_backward_adagrad_i64(plain, W, m, dev["grad"], dev["indices"].long(), bad_off, None,
                                     cfg.lr, cfg.eps, ws)
    assert e.value.status == tbe.TBE_ERR_INDEX_RANGE
    torch.cuda.synchronize()
    assert torch.equal(_bits(W), _bits(W0))


def _init_rows(n_rows, D, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    W = torch.empty((n_rows, D), dtype=dtype, device="cuda")
    W.uniform_(-0.01, 0.01, generator=g)
    return W


def _host_rows(W, keys):
    t = W.index_select(0, torch.from_numpy(keys.astype(np.int64)).cuda()).cpu()
    return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.slow
def test_rows_beyond_int32_total():
    """Three bf16 tables of 1.2e9, 1.0e9 and 0.5e9 rows (2.7e9 in total), D=8,
    B=4096, weighted; half the lookups on 64 hot rows near each table's end
    (long runs), half uniform over the table."""
    tbe = lib()
    rows = [1_200_000_000, 1_000_000_000, 500_000_000]
    T, D, B, dtype = 3, 8, 4096, "bf16"
    rng = np.random.default_rng(17)
    lengths = rng.poisson(20, T * B).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = int(offsets[-1])
    idx = np.empty(N, dtype=np.int64)
    for t in range(T):
        a, e = offsets[t * B], offsets[(t + 1) * B]
        n = int(e - a)
        hot = rows[t] - 1 - 997 * np.arange(64, dtype=np.int64)
        pick = rng.random(n) < 0.5
        idx[a:e] = np.where(pick, hot[rng.integers(0, 64, n)], rng.integers(0, rows[t], n))
    psw = rng.random(N).astype(np.float32)
    grad = rng.standard_normal((B, T * D)).astype(np.float32)
    roff = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    print(f"\n[int64] rows {sum(rows)} N={N}", flush=True)

    W = _init_rows(int(roff[-1]), D, torch.bfloat16, 3)
    m = torch.zeros(int(roff[-1]), dtype=torch.float32, device="cuda")
    touched = [np.unique(idx[offsets[t * B]:offsets[(t + 1) * B]]) for t in range(T)]
    W0 = [_host_rows(W, roff[t] + touched[t]) for t in range(T)]
    probe = np.concatenate([roff[t] + rng.integers(0, rows[t], 64) for t in range(T)])
    probe = np.setdiff1d(probe, np.concatenate([roff[t] + touched[t] for t in range(T)]))
    probe_before = _host_rows(W, probe)

    d_idx = torch.from_numpy(idx).cuda()
    d_off = torch.from_numpy(offsets).cuda()
    d_psw = torch.from_numpy(psw).cuda()
    d_grad = torch.from_numpy(grad).cuda()
    out = torch.empty((B, T * D), dtype=torch.float32, device="cuda")
    desc = tbe.Desc(T, D, B, rows, dtype)
    ws = tbe.workspace_i64(desc, N, True, tbe.TBE_OP_FORWARD)
    tbe.tbe_forward_i64(desc, W, d_idx, d_off, d_psw, out, ws)
    ws = tbe.workspace_i64(desc, N, True, tbe.TBE_OP_BACKWARD_SELF)
    tbe.tbe_backward_adagrad_i64(desc, W, m, d_grad, d_idx, d_off, d_psw, 0.01, 1e-8, ws)
    torch.cuda.synchronize()
    out_h = out.cpu().numpy()

    cfg = SimpleNamespace(dtype=dtype)
    for t in range(T):
        a, e = offsets[t * B], offsets[(t + 1) * B]
        keys_t = idx[a:e].astype(np.int32)            # in-table rows: below 2^31
        off_t = (offsets[t * B:(t + 1) * B + 1] - a).astype(np.int32)
        psw_t = psw[a:e]
        grad_t = np.ascontiguousarray(grad[:, t * D:(t + 1) * D])
        pre = oracle.preprocess(1, B, [rows[t]], keys_t, off_t, psw_t)
        ref = oracle.forward(1, B, D, dtype, off_t, pre["keys"], psw_t, W0[t], wkeys=touched[t])
        err = rel_err(out_h[:, t * D:(t + 1) * D], ref)
        assert err <= TOL[dtype], f"table {t}: forward rel err {err:.3g}"
        bw = oracle.backward_adagrad(1, B, D, dtype, pre["run_keys"], pre["run_offsets"],
                                     pre["sorted_bag"], pre["sorted_psw"], grad_t, W0[t],
                                     np.zeros(touched[t].size), 0.01, 1e-8, wkeys=touched[t])
        assert pre["long_runs"].size > 0
        assert_rows_match(cfg, W, m, roff[t] + pre["run_keys"].astype(np.int64), bw["w_new"],
                          bw["m_new"], f"table {t}")
    assert np.array_equal(_host_rows(W, probe), probe_before), "untouched rows changed"


@pytest.mark.slow
def test_lookups_beyond_int32_total():
    """2.2e9 lookups: two f32 tables of 1e6 and 1e8 rows, D=8, B=2^20 bags of
    1050 lookups. Lookup j of table t reads row (j * P) mod E_t with P =
    1,000,003 (prime to E_t), so row r is read by the lookups j = j0 + k*E_t,
    j0 = r * P^-1 mod E_t: 1101 lookups per row of table 0 (long runs), 11 per
    row of table 1 (short runs)."""
    tbe = lib()
    rows = [1_000_000, 100_000_000]
    T, D, B, L, P = 2, 8, 1 << 20, 1050, 1_000_003
    Nt = B * L
    N = T * Nt
    assert N >= 2 ** 31 and Nt < 2 ** 31 - 1
    print(f"\n[int64] N={N}", flush=True)
    idx = torch.empty(N, dtype=torch.int64, device="cuda")
    for t in range(T):
        seg = idx[t * Nt:(t + 1) * Nt]
        torch.arange(Nt, out=seg)
        seg.mul_(P).remainder_(rows[t])
    off = torch.arange(T * B + 1, dtype=torch.int64, device="cuda") * L
    roff = np.array([0, rows[0], rows[0] + rows[1]], dtype=np.int64)
    W = _init_rows(int(roff[-1]), D, torch.float32, 5)
    m = torch.zeros(int(roff[-1]), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(9)
    grad = torch.randn((B, T * D), generator=gen, device="cuda", dtype=torch.float32)
    grad_h = grad.cpu().numpy()
    rng = np.random.default_rng(21)
    sample_rows = [np.unique(np.concatenate([[0, rows[t] - 1], rng.integers(0, rows[t], 60)]))
                   for t in range(T)]
    sample_bags = np.sort(rng.choice(B, 200, replace=False))
    # weights the sampled bags read, and the sampled rows' own weights
    bag_rows = [((np.arange(L)[None, :] + L * sample_bags[:, None]) * P % rows[t]).astype(np.int64)
                for t in range(T)]
    need = [np.unique(np.concatenate([bag_rows[t].ravel(), sample_rows[t]])) for t in range(T)]
    W0 = [_host_rows(W, roff[t] + need[t]) for t in range(T)]

    out = torch.empty((B, T * D), dtype=torch.float32, device="cuda")
    desc = tbe.Desc(T, D, B, rows, "f32")
    ws = tbe.workspace_i64(desc, N, False, tbe.TBE_OP_FORWARD)
    print("[int64] forward", flush=True)
    tbe.tbe_forward_i64(desc, W, idx, off, None, out, ws)
    del ws
    torch.cuda.synchronize()
    ws = tbe.workspace_i64(desc, N, False, tbe.TBE_OP_BACKWARD_SELF)
    print(f"[int64] backward (workspace {ws.numel() / 1e9:.1f} GB)", flush=True)
    tbe.tbe_backward_adagrad_i64(desc, W, m, grad, idx, off, None, 0.01, 1e-8, ws)
    torch.cuda.synchronize()
    del ws
    out_h = out.cpu().numpy()

    cfg = SimpleNamespace(dtype="f32")
    for t in range(T):
        # forward on the sampled bags: a compact problem of those bags alone
        keys_s = bag_rows[t].ravel().astype(np.int32)
        off_s = (L * np.arange(sample_bags.size + 1)).astype(np.int32)
        ref = oracle.forward_bags(D, "f32", off_s, keys_s, None, W0[t],
                                  np.arange(sample_bags.size, dtype=np.int32), wkeys=need[t])
        got = out_h[sample_bags, t * D:(t + 1) * D]
        err = rel_err(got, ref)
        assert err <= TOL["f32"], f"table {t}: forward rel err {err:.3g}"
        # backward on the sampled rows: every lookup of each row, in batch order
        Pinv = pow(P, -1, rows[t])
        bags, counts = [], []
        for r in sample_rows[t]:
            js = (int(r) * Pinv) % rows[t] + rows[t] * np.arange((Nt - 1) // rows[t] + 2)
            js = js[js < Nt]
            bags.append((js // L).astype(np.int32))
            counts.append(js.size)
        run_offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        grad_t = np.ascontiguousarray(grad_h[:, t * D:(t + 1) * D])
        at = np.searchsorted(need[t], sample_rows[t])
        bw = oracle.backward_adagrad(1, B, D, "f32", sample_rows[t].astype(np.int32), run_offsets,
                                     np.concatenate(bags), None, grad_t, W0[t][at],
                                     np.zeros(sample_rows[t].size), 0.01, 1e-8,
                                     wkeys=sample_rows[t].astype(np.int32))
        print(f"[int64] table {t}: {counts[0]} lookups per sampled row", flush=True)
        assert_rows_match(cfg, W, m, roff[t] + sample_rows[t], bw["w_new"], bw["m_new"],
                          f"table {t}")
