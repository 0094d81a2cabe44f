"""Pins of the CPU oracle against things other than itself: brute force on tiny
inputs, library routines (numpy, torch.nn.functional.embedding_bag,
torch.optim.Adagrad), closed forms and invariants. CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import (bag_major_to_out, incidence, tiny_problem,
                           weights_as_f64)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SEEDS = list(range(12))


def _prep(p, S=256, C=256):
    return oracle.preprocess(p["T"], p["B"], p["rows"], p["indices"], p["offsets"],
                             p["psw"], S, C)


# --------------------------------------------------------------------------
# Linearize / validation
# --------------------------------------------------------------------------

def test_linearize_matches_table_offsets_and_bags():
    rng = np.random.default_rng(0)
    p = tiny_problem(rng, T=3, B=5, rows=[7, 11, 5])
    keys, bags = oracle.linearize(p["T"], p["B"], p["rows"], p["indices"], p["offsets"])
    first = np.array([0, 7, 18])
    lengths = np.diff(p["offsets"])
    exp_bags = np.repeat(np.arange(p["T"] * p["B"]), lengths)
    np.testing.assert_array_equal(bags, exp_bags)
    np.testing.assert_array_equal(keys, first[exp_bags // p["B"]] + p["indices"])


@pytest.mark.parametrize("bad", ["index_high", "index_neg", "offsets_dec", "offsets_end"])
def test_linearize_rejects_bad_input(bad):
    rng = np.random.default_rng(1)
    p = tiny_problem(rng, T=2, B=4, rows=[5, 5], empty_frac=0.0, max_len=3)
    idx, off = p["indices"].copy(), p["offsets"].copy()
    if bad == "index_high":
        idx[-1] = 5
    elif bad == "index_neg":
        idx[0] = -1
    elif bad == "offsets_dec":
        off[2], off[3] = off[3], off[2] - 1
    else:
        off[-1] += 1
    with pytest.raises(oracle.OracleError):
        oracle.linearize(2, 4, [5, 5], idx, off)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_forward_equals_dense_incidence_product(seed, dtype):
    rng = np.random.default_rng(seed)
    p = tiny_problem(rng, dtype=dtype)
    keys, _ = oracle.linearize(p["T"], p["B"], p["rows"], p["indices"], p["offsets"])
    out = oracle.forward(p["T"], p["B"], p["D"], dtype, p["offsets"], keys, p["psw"], p["W"])
    A = incidence(p)
    ref = bag_major_to_out(A @ weights_as_f64(p["W"], dtype), p["T"], p["B"], p["D"])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", SEEDS[:6])
def test_forward_equals_torch_embedding_bag(seed):
    rng = np.random.default_rng(100 + seed)
    p = tiny_problem(rng, dtype="f32")
    keys, _ = oracle.linearize(p["T"], p["B"], p["rows"], p["indices"], p["offsets"])
    out = oracle.forward(p["T"], p["B"], p["D"], "f32", p["offsets"], keys, p["psw"], p["W"])
    W = torch.from_numpy(p["W"].astype(np.float64))
    first = np.concatenate([[0], np.cumsum(p["rows"])[:-1]])
    T, B, D = p["T"], p["B"], p["D"]
    for t in range(T):
        a, b = p["offsets"][t * B], p["offsets"][(t + 1) * B]
        off = torch.from_numpy((p["offsets"][t * B:(t + 1) * B] - a).astype(np.int64))
        idx = torch.from_numpy(p["indices"][a:b].astype(np.int64))
        psw = None if p["psw"] is None else torch.from_numpy(p["psw"][a:b].astype(np.float64))
        Wt = W[first[t]:first[t] + p["rows"][t]]
        ref = torch.nn.functional.embedding_bag(idx, Wt, off, mode="sum",
                                                per_sample_weights=psw)
        np.testing.assert_allclose(out[:, t * D:(t + 1) * D], ref.numpy(), rtol=1e-12, atol=1e-15)


def test_forward_single_lookup_bags_are_row_gathers():
    rng = np.random.default_rng(7)
    p = tiny_problem(rng, T=2, B=9, D=16, rows=[30, 40], weighted=False, empty_frac=0.0,
                     max_len=1)
    p["offsets"] = np.arange(p["T"] * p["B"] + 1, dtype=np.int32)
    p["indices"] = rng.integers(0, 30, size=p["T"] * p["B"]).astype(np.int32)
    keys, _ = oracle.linearize(2, 9, p["rows"], p["indices"], p["offsets"])
    out = oracle.forward(2, 9, 16, "f32", p["offsets"], keys, None, p["W"])
    ref = bag_major_to_out(p["W"][keys].astype(np.float64), 2, 9, 16)
    np.testing.assert_array_equal(out, ref)


def test_forward_empty_bags_are_zero_and_row_store_subset_agrees():
    rng = np.random.default_rng(8)
    p = tiny_problem(rng, T=2, B=8, D=3, rows=[20, 20], empty_frac=0.5)
    keys, _ = oracle.linearize(2, 8, p["rows"], p["indices"], p["offsets"])
    out = oracle.forward(2, 8, 3, "f32", p["offsets"], keys, p["psw"], p["W"])
    lengths = np.diff(p["offsets"]).reshape(2, 8)
    for t in range(2):
        for b in range(8):
            if lengths[t, b] == 0:
                assert not out[b, t * 3:(t + 1) * 3].any()
    uk = np.unique(keys)
    sub = oracle.forward(2, 8, 3, "f32", p["offsets"], keys, p["psw"], p["W"][uk], wkeys=uk)
    np.testing.assert_array_equal(sub, out)


# --------------------------------------------------------------------------
# Sort / RLE
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", SEEDS)
def test_sort_and_rle_match_numpy(seed):
    rng = np.random.default_rng(200 + seed)
    p = tiny_problem(rng, max_len=12)
    r = _prep(p)
    keys = r["keys"]
    np.testing.assert_array_equal(r["sorted_pos"], np.argsort(keys, kind="stable"))
    uk, first, counts = np.unique(keys, return_index=True, return_counts=True)
    np.testing.assert_array_equal(r["run_keys"], uk)
    np.testing.assert_array_equal(np.diff(r["run_offsets"]), counts)
    assert r["run_offsets"][0] == 0 and r["run_offsets"][-1] == keys.size
    np.testing.assert_array_equal(r["sorted_bag"], r["bags"][r["sorted_pos"]])
    if p["psw"] is not None:
        np.testing.assert_array_equal(r["sorted_psw"], p["psw"][r["sorted_pos"]])


def test_sort_invariants_on_skewed_keys():
    rng = np.random.default_rng(5)
    keys = (rng.zipf(1.3, size=20000) % 3000).astype(np.int32)
    pos = oracle.sort(keys)
    assert np.array_equal(np.sort(pos), np.arange(keys.size))           # permutation
    ks = keys[pos]
    assert np.all(np.diff(ks) >= 0)                                      # sorted
    same = np.diff(ks) == 0
    assert np.all(np.diff(pos)[same] > 0)                                # stable ties


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------

def test_route_boundaries_at_256_and_512():
    sls = [255, 256, 257, 511, 512, 513, 1, 0 + 2]
    ro = np.concatenate([[0], np.cumsum(sls)]).astype(np.int32)
    r = oracle.route(ro, S=256, C=256)
    np.testing.assert_array_equal(r["short_runs"], [0, 6, 7])
    np.testing.assert_array_equal(r["long_runs"], [1, 2, 3, 4, 5])
    # chunks: 256 -> 1, 257 -> 2, 511 -> 2, 512 -> 2, 513 -> 3
    np.testing.assert_array_equal(r["chunk_run"], [1, 2, 2, 3, 3, 4, 4, 5, 5, 5])
    starts = [ro[1], ro[2], ro[2] + 256, ro[3], ro[3] + 256, ro[4], ro[4] + 256,
              ro[5], ro[5] + 256, ro[5] + 512]
    np.testing.assert_array_equal(r["chunk_start"], starts)
    np.testing.assert_array_equal(r["long_chunk_begin"], [0, 1, 3, 5, 7, 10])


@pytest.mark.parametrize("S,C", [(256, 256), (4, 3), (1, 1), (10, 64)])
def test_route_partitions_runs_and_chunks(S, C):
    rng = np.random.default_rng(S * 1000 + C)
    sls = rng.integers(1, 700, size=300)
    ro = np.concatenate([[0], np.cumsum(sls)]).astype(np.int32)
    r = oracle.route(ro, S=S, C=C)
    allr = np.sort(np.concatenate([r["short_runs"], r["long_runs"]]))
    np.testing.assert_array_equal(allr, np.arange(300))
    assert np.all(sls[r["short_runs"]] < S) and np.all(sls[r["long_runs"]] >= S)
    assert np.all(np.diff(r["short_runs"]) > 0) and np.all(np.diff(r["long_runs"]) > 0)
    covered = np.zeros(ro[-1], dtype=np.int64)
    for c in range(r["chunk_run"].size):
        u = r["chunk_run"][c]
        a = r["chunk_start"][c]
        e = min(a + C, ro[u + 1])
        assert ro[u] <= a < ro[u + 1]
        covered[a:e] += 1
    long_mask = np.zeros(ro[-1], dtype=bool)
    for u in r["long_runs"]:
        long_mask[ro[u]:ro[u + 1]] = True
    assert np.all(covered[long_mask] == 1) and np.all(covered[~long_mask] == 0)


# --------------------------------------------------------------------------
# Backward: per-run gradient
# --------------------------------------------------------------------------

def _backward(p, m=None, lr=0.01, eps=1e-8, want_g=True):
    r = _prep(p)
    if m is None:
        m = np.zeros(p["E"], dtype=np.float32)
    res = oracle.backward_adagrad(p["T"], p["B"], p["D"], p["dtype"], r["run_keys"],
                                  r["run_offsets"], r["sorted_bag"], r["sorted_psw"],
                                  p["grad"], p["W"], m, lr, eps, want_g=want_g)
    return r, res


@pytest.mark.parametrize("seed", SEEDS)
def test_run_gradient_equals_incidence_transpose_product(seed):
    rng = np.random.default_rng(300 + seed)
    p = tiny_problem(rng)
    r, res = _backward(p)
    A = incidence(p)
    T, B, D = p["T"], p["B"], p["D"]
    G_bag = p["grad"].astype(np.float64).reshape(B, T, D).transpose(1, 0, 2).reshape(T * B, D)
    G = A.T @ G_bag
    np.testing.assert_allclose(res["g"], G[r["run_keys"]], rtol=1e-12, atol=1e-14)
    touched = np.zeros(p["E"], dtype=bool)
    touched[r["run_keys"]] = True
    assert np.array_equal(touched, np.abs(A).sum(axis=0) > 0)


def test_gradient_mass_conservation_per_table():
    rng = np.random.default_rng(9)
    p = tiny_problem(rng, T=3, B=16, D=16, weighted=True, max_len=10)
    r, res = _backward(p)
    T, B, D = 3, 16, 16
    first = np.concatenate([[0], np.cumsum(p["rows"])])
    lengths_w = np.zeros(T * B)
    for i in range(T * B):
        lengths_w[i] = p["psw"][p["offsets"][i]:p["offsets"][i + 1]].astype(np.float64).sum()
    for t in range(T):
        sel = (r["run_keys"] >= first[t]) & (r["run_keys"] < first[t + 1])
        lhs = res["g"][sel].sum(axis=0)
        rows = p["grad"][:, t * D:(t + 1) * D].astype(np.float64)
        rhs = (lengths_w[t * B:(t + 1) * B, None] * rows).sum(axis=0)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-12)


def test_constant_gradient_gives_segment_length_times_constant():
    rng = np.random.default_rng(10)
    p = tiny_problem(rng, T=2, B=12, D=3, weighted=False, max_len=9)
    p["grad"][:] = np.float32(0.375)
    r, res = _backward(p)
    sl = np.diff(r["run_offsets"]).astype(np.float64)
    np.testing.assert_array_equal(res["g"], np.repeat(sl[:, None] * 0.375, 3, axis=1))


# --------------------------------------------------------------------------
# Row-wise Adagrad
# --------------------------------------------------------------------------

def test_adagrad_closed_form_for_rows_touched_once():
    rng = np.random.default_rng(11)
    T, B, D = 1, 40, 16
    E = 100
    keys = rng.permutation(E)[:B]                                      # distinct rows
    p = dict(T=T, B=B, D=D, rows=[E], dtype="f32", E=E,
             indices=keys.astype(np.int32), offsets=np.arange(B + 1, dtype=np.int32),
             psw=rng.random(B).astype(np.float32),
             W=rng.uniform(-0.01, 0.01, (E, D)).astype(np.float32),
             grad=rng.standard_normal((B, D)).astype(np.float32))
    r, res = _backward(p)
    lr, eps = 0.01, 1e-8
    for u, key in enumerate(r["run_keys"]):
        b = int(np.nonzero(keys == key)[0][0])
        g = np.float64(p["psw"][b]) * p["grad"][b].astype(np.float64)
        rms = np.sqrt(np.mean(g * g))
        np.testing.assert_allclose(res["m_new"][u], np.mean(g * g), rtol=1e-14)
        np.testing.assert_allclose(res["w_new"][u], p["W"][key] - lr * g / (rms + eps),
                                   rtol=1e-13, atol=1e-17)


@pytest.mark.parametrize("seed", range(6))
def test_adagrad_one_column_equals_torch_adagrad_two_steps(seed):
    """D = 1: row-wise Adagrad is torch.optim.Adagrad on a dense gradient, and
    the per-row sum of all lookups gets a single update (not one per lookup)."""
    rng = np.random.default_rng(400 + seed)
    p = tiny_problem(rng, D=1, dtype="f32", max_len=10)
    lr, eps = 0.05, 1e-8
    m0 = rng.random(p["E"]).astype(np.float32)
    W0 = p["W"].astype(np.float64)
    param = torch.nn.Parameter(torch.from_numpy(W0.copy()))
    opt = torch.optim.Adagrad([param], lr=lr, eps=eps, lr_decay=0, weight_decay=0,
                              initial_accumulator_value=0.0)
    opt.state[param]["sum"] = torch.from_numpy(m0.astype(np.float64)[:, None].copy())
    opt.state[param]["step"] = torch.tensor(0.0)
    A = incidence(p)
    T, B = p["T"], p["B"]
    G_bag = p["grad"].astype(np.float64).reshape(B, T, 1).transpose(1, 0, 2).reshape(T * B, 1)
    W_cur, m_cur = p["W"].copy(), m0.copy()
    for step in range(2):
        param.grad = torch.from_numpy(A.T @ G_bag)
        opt.step()
        q = dict(p, W=W_cur)
        r, res = _backward(q, m=m_cur, lr=lr, eps=eps)
        ref = param.detach().numpy()[:, 0]
        np.testing.assert_allclose(res["w_new"][:, 0], ref[r["run_keys"]], rtol=1e-6, atol=1e-9)
        np.testing.assert_allclose(res["m_new"], opt.state[param]["sum"].numpy()[r["run_keys"], 0],
                                   rtol=1e-6)
        # carry the oracle's state forward exactly as the device would store it
        W_cur = W_cur.copy()
        W_cur[r["run_keys"], 0] = oracle.round_to(res["w_new"][:, 0], "f32").astype(np.float32)
        m_cur = m_cur.copy()
        m_cur[r["run_keys"]] = oracle.round_to(res["m_new"], "f32").astype(np.float32)
        param.data[:, 0] = torch.from_numpy(W_cur[:, 0].astype(np.float64))
        opt.state[param]["sum"][:, 0] = torch.from_numpy(m_cur.astype(np.float64))


def test_adagrad_constant_columns_equals_elementwise_torch_adagrad():
    """When every column of a row's gradient is equal, the row mean of g^2 is
    each element's g^2, so row-wise Adagrad is element-wise Adagrad for D > 1."""
    rng = np.random.default_rng(12)
    T, B, D = 2, 10, 16
    p = tiny_problem(rng, T=T, B=B, D=D, dtype="f32", max_len=6, weighted=True)
    col = rng.standard_normal((B, T, 1)).astype(np.float32)
    p["grad"] = np.ascontiguousarray(np.broadcast_to(col, (B, T, D)).reshape(B, T * D))
    m0 = rng.random(p["E"]).astype(np.float32)
    lr, eps = 0.01, 1e-8
    r, res = _backward(p, m=m0, lr=lr, eps=eps)
    param = torch.nn.Parameter(torch.from_numpy(p["W"].astype(np.float64)))
    opt = torch.optim.Adagrad([param], lr=lr, eps=eps)
    opt.state[param]["sum"] = torch.from_numpy(np.repeat(m0.astype(np.float64)[:, None], D, 1))
    opt.state[param]["step"] = torch.tensor(0.0)
    A = incidence(p)
    G_bag = p["grad"].astype(np.float64).reshape(B, T, D).transpose(1, 0, 2).reshape(T * B, D)
    param.grad = torch.from_numpy(A.T @ G_bag)
    opt.step()
    ref = param.detach().numpy()[r["run_keys"]]
    np.testing.assert_allclose(res["w_new"], ref, rtol=1e-10, atol=1e-14)


def test_untouched_rows_are_not_emitted_and_zero_gradient_run_is_still_a_run():
    rng = np.random.default_rng(13)
    p = tiny_problem(rng, T=1, B=6, D=4, rows=[30], weighted=False)
    p["grad"][:] = 0.0
    m0 = np.full(p["E"], 0.25, dtype=np.float32)
    r, res = _backward(p, m=m0)
    assert set(r["run_keys"]) == set(np.unique(r["keys"]))
    np.testing.assert_array_equal(res["m_new"], 0.25)
    np.testing.assert_array_equal(res["w_new"], p["W"][r["run_keys"]].astype(np.float64))


# --------------------------------------------------------------------------
# Small-table counts
# --------------------------------------------------------------------------

def test_histogram_matches_bincount_and_bag_lengths():
    rng = np.random.default_rng(14)
    T, B, E = 3, 20, 64
    lengths = rng.integers(0, 100, size=T * B)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    indices = rng.integers(0, E, size=offsets[-1]).astype(np.int32)
    H = oracle.histogram(T, B, E, [E] * T, indices, offsets)
    for i in range(T * B):
        ref = np.bincount(indices[offsets[i]:offsets[i + 1]], minlength=E)
        np.testing.assert_array_equal(H.reshape(T * B, E)[i], ref)
    np.testing.assert_array_equal(H.sum(axis=2).reshape(-1), lengths)


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 6.1e-5, 5.96e-8, 2.98e-8,
            2.9802322e-08, 1e-40, 3.4e38, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 1.0 + 2 ** -8,
            1.0 + 3 * 2 ** -8, 2 ** -126, 2 ** -133, np.inf, -np.inf]
    return np.array(vals, dtype=np.float32)


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(15)
    bits = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = np.concatenate([x, _special_f32(), rng.standard_normal(100000).astype(np.float32)])
    got = oracle.round_to(x.astype(np.float64), "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(got, ref)
    # doubles (not representable in f32) against numpy's direct double->half
    d = rng.standard_normal(100000) * 10.0 ** rng.integers(-9, 5, size=100000)
    with np.errstate(over="ignore"):
        np.testing.assert_array_equal(oracle.round_to(d, "f16"), d.astype(np.float16).astype(np.float64))


def test_round_bf16_matches_torch_on_f32_inputs():
    rng = np.random.default_rng(16)
    bits = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = np.concatenate([x, _special_f32()])
    got = oracle.round_to(x.astype(np.float64), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)


def test_round_f32_matches_numpy_cast():
    rng = np.random.default_rng(17)
    d = rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, size=200000)
    with np.errstate(over="ignore"):
        ref = d.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_to(d, "f32"), ref)


def test_decode_matches_numpy_and_torch():
    bits = np.arange(2 ** 16, dtype=np.uint16)
    h = oracle.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    same = (h == ref) | (np.isnan(h) & np.isnan(ref))
    assert same.all()
    b = oracle.decode(bits, "bf16")
    refb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    sameb = (b == refb) | (np.isnan(b) & np.isnan(refb))
    assert sameb.all()


# --------------------------------------------------------------------------
# Golden: the page's stated thresholds are the ones the oracle routes with
# --------------------------------------------------------------------------

def test_route_default_threshold_is_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "page1_thresholds.json")))
    S, C = g["short_max"], g["chunk"]
    ro = np.array([0, S - 1, 2 * S - 1, 2 * S - 1 + 2 * C + 1], dtype=np.int32)
    r = oracle.route(ro, S=S, C=C)
    np.testing.assert_array_equal(r["short_runs"], [0])
    np.testing.assert_array_equal(r["long_runs"], [1, 2])
    np.testing.assert_array_equal(r["long_chunk_begin"], [0, 1, 4])


def test_compensated_f16_split_error_bound():
    """The small-table backward contracts the f32 upstream gradient as two f16
    halves, hi = f16(g) and lo = f16((g - hi) * 2^11) (the page's compensated
    f16 high/low product to f32). Their sum recovers g to about 2^-22
    relative: hi is within 2^-11 of g, the residual g - hi is exact in f32,
    and lo carries it with another 2^-11 relative error (plus a subnormal
    floor of 2^-25 / 2^11 = 2^-36 absolute). Checked with numpy's own f16
    rounding, independent of the library, over the f16 normal range and at
    the range's end, where hi overflows and the split no longer holds."""
    rng = np.random.default_rng(2024)
    mag = np.exp2(rng.uniform(-14.0, np.log2(65504.0), 400_000))
    g = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    g = np.concatenate([g, np.float32([1.0, -1.0, 65504.0, -65504.0, 2.0 ** -14, 3.0e-5,
                                       np.nextafter(np.float32(65504.0), np.float32(0))])])
    hi = g.astype(np.float16)
    r = g - hi.astype(np.float32)                       # exact in f32
    lo = (r * np.float32(2048.0)).astype(np.float16)
    back = hi.astype(np.float64) + lo.astype(np.float64) / 2048.0
    err = np.abs(back - g.astype(np.float64))
    assert np.all(np.isfinite(hi)) and np.all(np.isfinite(lo))
    assert np.all(err <= 2.0 ** -22 * np.abs(g.astype(np.float64)) + 2.0 ** -36)
    # the bound is tight to within a factor of a few: a plain f16 rounding of
    # g alone is 2^11 times worse, so the lo half is doing the work
    assert np.median(err / np.abs(g)) < 2.0 ** -24
    plain = np.abs(hi.astype(np.float64) - g)
    assert np.median(plain / np.abs(g)) > 2.0 ** -14
    # beyond f16's largest finite value the high half overflows: such
    # gradients cannot take this path (the library redoes them in f32)
    big = np.float32([65520.0, 1.0e5, -3.0e9])
    with np.errstate(over="ignore"):
        assert np.all(np.isinf(big.astype(np.float16)))
