"""Property-based pins of the CPU oracle (hypothesis): on generated jagged
batches (empty bags, repeated rows inside and across bags, single-row tables,
D in {1, 3, 16, 128}, weighted and unweighted, f32/f16/bf16 weights) the
oracle must agree with definitions computed another way: the dense incidence
matrix for the forward and the per-row gradient, numpy's stable argsort and
unique for the transpose, a plain loop for the routing, and the row-wise
shape of the optimizer update. CPU only."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from tests.helpers import bag_major_to_out, incidence, weights_as_f64

SETTINGS = settings(max_examples=40, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def batches(draw):
    T = draw(st.integers(1, 3))
    B = draw(st.integers(1, 12))
    D = draw(st.sampled_from([1, 3, 16, 128]))
    rows = [draw(st.integers(1, 40)) for _ in range(T)]
    weighted = draw(st.booleans())
    dtype = draw(st.sampled_from(["f32", "f16", "bf16"]))
    max_len = draw(st.integers(0, 10))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, max_len + 1, size=T * B)
    lengths[rng.random(T * B) < 0.25] = 0
    offsets = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    N = int(offsets[-1])
    indices = np.empty(N, dtype=np.int32)
    for t in range(T):
        a, b = offsets[t * B], offsets[(t + 1) * B]
        hot = rng.integers(0, rows[t], size=max(1, rows[t] // 4))  # rows repeat
        indices[a:b] = rng.choice(hot, size=b - a)
    psw = rng.random(N).astype(np.float32) if weighted else None
    E = int(sum(rows))
    Wf = rng.uniform(-0.01, 0.01, size=(E, D)).astype(np.float32)
    if dtype == "f32":
        W = Wf
    elif dtype == "f16":
        W = Wf.astype(np.float16).view(np.uint16)
    else:
        import torch
        W = torch.from_numpy(Wf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    grad = rng.standard_normal((B, T * D)).astype(np.float32)
    S = draw(st.integers(1, 6))
    C = draw(st.integers(1, 5))
    return dict(T=T, B=B, D=D, rows=rows, dtype=dtype, indices=indices,
                offsets=offsets.astype(np.int32), psw=psw, W=W, grad=grad, E=E, S=S, C=C)


@SETTINGS
@given(batches())
def test_forward_is_the_incidence_product(p):
    keys, _ = oracle.linearize(p["T"], p["B"], p["rows"], p["indices"], p["offsets"])
    out = oracle.forward(p["T"], p["B"], p["D"], p["dtype"], p["offsets"], keys, p["psw"], p["W"])
    ref = bag_major_to_out(incidence(p) @ weights_as_f64(p["W"], p["dtype"]),
                           p["T"], p["B"], p["D"])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)


@SETTINGS
@given(batches())
def test_transpose_is_a_stable_sort_and_its_runs(p):
    r = oracle.preprocess(p["T"], p["B"], p["rows"], p["indices"], p["offsets"], p["psw"],
                          p["S"], p["C"])
    keys = np.asarray(r["keys"])
    order = np.argsort(keys, kind="stable")
    assert np.array_equal(r["sorted_pos"], order)
    uk, counts = np.unique(keys, return_counts=True)
    assert np.array_equal(r["run_keys"], uk)
    assert np.array_equal(r["run_offsets"], np.concatenate([[0], np.cumsum(counts)]))
    # the bag of every lookup, from the offsets by brute force
    bag_of = np.repeat(np.arange(p["T"] * p["B"]), np.diff(p["offsets"]))
    assert np.array_equal(r["sorted_bag"], bag_of[order])
    if p["psw"] is None:
        assert r["sorted_psw"] is None  # unweighted: no weight copy is made
    else:
        assert np.array_equal(r["sorted_psw"], p["psw"][order])


@SETTINGS
@given(batches())
def test_routing_partitions_runs_and_chunks(p):
    r = oracle.preprocess(p["T"], p["B"], p["rows"], p["indices"], p["offsets"], p["psw"],
                          p["S"], p["C"])
    S, C = p["S"], p["C"]
    ro = np.asarray(r["run_offsets"])
    short, long_, cr, cs = [], [], [], []
    for u in range(ro.size - 1):
        sl = ro[u + 1] - ro[u]
        if sl < S:
            short.append(u)
        else:
            long_.append(u)
            for k in range(ro[u], ro[u + 1], C):
                cr.append(u)
                cs.append(k)
    assert np.array_equal(r["short_runs"], np.array(short, dtype=np.int32))
    assert np.array_equal(r["long_runs"], np.array(long_, dtype=np.int32))
    assert np.array_equal(r["chunk_run"], np.array(cr, dtype=np.int32))
    assert np.array_equal(r["chunk_start"], np.array(cs, dtype=np.int32))


@SETTINGS
@given(batches())
def test_run_gradient_and_row_wise_update(p):
    r = oracle.preprocess(p["T"], p["B"], p["rows"], p["indices"], p["offsets"], p["psw"])
    rng = np.random.default_rng(len(r["run_keys"]))
    m = rng.uniform(0.0, 1.0, size=p["E"]).astype(np.float32)
    res = oracle.backward_adagrad(p["T"], p["B"], p["D"], p["dtype"], r["run_keys"],
                                  r["run_offsets"], r["sorted_bag"], r["sorted_psw"], p["grad"],
                                  p["W"], m, 0.01, 1e-8, want_g=True)
    T, B, D = p["T"], p["B"], p["D"]
    G_bag = p["grad"].astype(np.float64).reshape(B, T, D).transpose(1, 0, 2).reshape(T * B, D)
    G = incidence(p).T @ G_bag
    keys = np.asarray(r["run_keys"])
    np.testing.assert_allclose(res["g"], G[keys], rtol=1e-12, atol=1e-14)
    # state only grows; the step is -g times one positive factor per row
    m_old = m[keys].astype(np.float64)
    assert np.all(res["m_new"] >= m_old)
    w_old = weights_as_f64(p["W"], p["dtype"])[keys]
    step = res["w_new"] - w_old
    g = res["g"]
    for u in range(keys.size):
        nz = g[u] != 0
        if not nz.any():
            assert np.all(step[u] == 0)
            continue
        ratio = -step[u][nz] / g[u][nz]
        assert np.all(ratio > 0)
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-9)
