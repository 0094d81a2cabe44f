"""Test-side helpers: the error metric, tiny random problems and dense
reference constructions used to pin the oracle."""
from __future__ import annotations

import numpy as np


def rel_err(x, y) -> float:
    """max_i |x_i - y_i| / max(|y_i|, rms of y's row): relative error with a
    per-row floor so that elements near zero do not dominate. `y` is the
    reference (the oracle's unrounded value)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if y.size == 0:
        return 0.0
    y2 = y.reshape(y.shape[0], -1) if y.ndim > 1 else y.reshape(-1, 1)
    x2 = x.reshape(y2.shape)
    rms = np.sqrt(np.mean(y2 * y2, axis=1, keepdims=True))
    denom = np.maximum(np.abs(y2), rms)
    denom = np.where(denom == 0, 1.0, denom)
    return float(np.max(np.abs(x2 - y2) / denom))


TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}


def tiny_problem(rng, T=None, B=None, D=None, dtype="f32", weighted=None,
                 max_len=8, rows=None, empty_frac=0.2):
    """A small jagged batch with empty bags and repeated rows inside bags."""
    T = int(rng.integers(1, 4)) if T is None else T
    B = int(rng.integers(1, 17)) if B is None else B
    D = int(rng.choice([1, 3, 16])) if D is None else D
    if rows is None:
        rows = [int(rng.integers(1, 51)) for _ in range(T)]
    weighted = bool(rng.integers(0, 2)) if weighted is None else weighted
    lengths = rng.integers(0, max_len + 1, size=T * B)
    lengths[rng.random(T * B) < empty_frac] = 0
    offsets = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    N = int(offsets[-1])
    indices = np.empty(N, dtype=np.int32)
    for t in range(T):
        a, b = offsets[t * B], offsets[(t + 1) * B]
        # few distinct rows so that rows repeat inside and across bags
        hot = rng.integers(0, rows[t], size=max(1, rows[t] // 3))
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
    return dict(T=T, B=B, D=D, rows=rows, dtype=dtype, indices=indices,
                offsets=offsets.astype(np.int32), psw=psw, W=W, grad=grad, E=E)


def weights_as_f64(W, dtype):
    """Values of raw weights via numpy/torch (independent of the oracle)."""
    if dtype == "f32":
        return np.asarray(W, dtype=np.float64)
    if dtype == "f16":
        return np.asarray(W).view(np.float16).astype(np.float64)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def incidence(p):
    """Dense A[i, key] = sum of per-sample weights of the lookups of bag i on
    stacked row `key` (bag i = t*B + b)."""
    T, B, rows = p["T"], p["B"], p["rows"]
    first = np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(np.int64)
    A = np.zeros((T * B, int(sum(rows))), dtype=np.float64)
    off = p["offsets"]
    for i in range(T * B):
        t = i // B
        for j in range(off[i], off[i + 1]):
            s = 1.0 if p["psw"] is None else float(p["psw"][j])
            A[i, first[t] + p["indices"][j]] += s
    return A


def bag_major_to_out(P, T, B, D):
    """[T*B, D] per-bag rows (bag i = t*B + b) to the [B, T*D] output layout."""
    return P.reshape(T, B, D).transpose(1, 0, 2).reshape(B, T * D)


def out_to_bag_major(O, T, B, D):
    return O.reshape(B, T, D).transpose(1, 0, 2).reshape(T * B, D)
