"""CPU oracle for the TBE hot path: ctypes wrapper over tbe_oracle.c.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package. It shares no code
with the HIP library. Every step follows the FBTriton TBE tutorial (page 1):
linearize, pool, stable sort, run-length encode, route by segment length,
per-run gradient sum, one row-wise Adagrad step per touched row; plus the
small-table per-bag counts. The C file's header states each definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tbe_oracle.c")
_LIB = os.path.join(_HERE, "libtbe_oracle.so")
# A test that plants mistakes in a copy of the C source points this at the
# mutant build; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("TBE_ORACLE_LIB")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
ERRORS = {0: "ok", 1: "bad argument", 2: "bad offsets", 3: "index out of range",
          4: "row missing from store", 5: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build(force=False)
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.or_round.restype = dbl
        L.or_round.argtypes = [dbl, ctypes.c_int]
        L.or_round_array.argtypes = [P, i64, ctypes.c_int, P]
        L.or_decode_array.argtypes = [P, i64, ctypes.c_int, P]
        L.or_linearize.argtypes = [i32, i32, P, i64, P, P, P, P]
        L.or_forward_bags.argtypes = [i32, ctypes.c_int, P, P, P, P, i64, P, i64, P, P]
        L.or_forward.argtypes = [i32, i32, i32, ctypes.c_int, P, P, P, P, i64, P, P]
        L.or_sort.argtypes = [i64, P, P]
        L.or_rle.restype = i64
        L.or_rle.argtypes = [i64, P, P, P, P, P, P, P, P]
        L.or_route.argtypes = [i64, P, i32, i32, P, P, P, P, P, P]
        L.or_backward_adagrad.argtypes = [i32, i32, i32, ctypes.c_int, i64, P, P, P, P, P,
                                          P, i64, P, P, dbl, dbl, P, P, P]
        L.or_histogram.argtypes = [i32, i32, i32, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc):
    if rc != 0:
        raise OracleError(ERRORS.get(rc, f"error {rc}"))


# --- number formats ---------------------------------------------------------

def round_to(x, dtype: str) -> np.ndarray:
    """Round doubles to the nearest f32/f16/bf16 value (ties to even); the
    result is returned as doubles holding exactly representable values."""
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib().or_round_array(_p(x), x.size, DTYPES[dtype], _p(y))
    return y


def decode(raw, dtype: str) -> np.ndarray:
    """Values of raw storage: float32 array, or uint16 bit patterns for f16/bf16."""
    raw = np.ascontiguousarray(raw)
    y = np.empty(raw.size, dtype=np.float64)
    lib().or_decode_array(_p(raw), raw.size, DTYPES[dtype], _p(y))
    return y.reshape(raw.shape)


def _raw_weights(W, dtype):
    """float32 array for f32; uint16 bit patterns for f16/bf16."""
    W = np.ascontiguousarray(W)
    if dtype == "f32":
        assert W.dtype == np.float32
        return W
    assert W.dtype in (np.uint16, np.int16), "f16/bf16 weights are passed as raw bits"
    return W.view(np.uint16)


# --- the method's steps -------------------------------------------------------

def linearize(T, B, rows, indices, offsets):
    indices = _c(indices, np.int32)
    offsets = _c(offsets, np.int32)
    rows = _c(rows, np.int64)
    N = indices.size
    keys = np.empty(N, dtype=np.int32)
    bags = np.empty(N, dtype=np.int32)
    _check(lib().or_linearize(T, B, _p(rows), N, _p(indices), _p(offsets), _p(keys), _p(bags)))
    return keys, bags


def forward(T, B, D, dtype, offsets, keys, psw, W, wkeys=None):
    """Pooled output [B, T*D] as doubles. W holds rows for `wkeys` (sorted) or
    every stacked row when wkeys is None."""
    offsets, keys, psw = _c(offsets, np.int32), _c(keys, np.int32), _c(psw, np.float32)
    raw = _raw_weights(W, dtype)
    wk = _c(wkeys, np.int32)
    out = np.empty((B, T * D), dtype=np.float64)
    _check(lib().or_forward(T, B, D, DTYPES[dtype], _p(offsets), _p(keys), _p(psw),
                            _p(wk), 0 if wk is None else wk.size, _p(raw), _p(out)))
    return out


def forward_bags(D, dtype, offsets, keys, psw, W, bag_ids, wkeys=None):
    offsets, keys, psw = _c(offsets, np.int32), _c(keys, np.int32), _c(psw, np.float32)
    raw = _raw_weights(W, dtype)
    wk = _c(wkeys, np.int32)
    bag_ids = _c(bag_ids, np.int32)
    out = np.empty((bag_ids.size, D), dtype=np.float64)
    _check(lib().or_forward_bags(D, DTYPES[dtype], _p(offsets), _p(keys), _p(psw), _p(wk),
                                 0 if wk is None else wk.size, _p(raw), bag_ids.size,
                                 _p(bag_ids), _p(out)))
    return out


def sort(keys):
    keys = _c(keys, np.int32)
    pos = np.empty(keys.size, dtype=np.int32)
    _check(lib().or_sort(keys.size, _p(keys), _p(pos)))
    return pos


def rle(keys, sorted_pos, bags, psw):
    keys, sorted_pos, bags = _c(keys, np.int32), _c(sorted_pos, np.int32), _c(bags, np.int32)
    psw = _c(psw, np.float32)
    N = keys.size
    run_keys = np.empty(N, dtype=np.int32)
    run_offsets = np.empty(N + 1, dtype=np.int32)
    sorted_bag = np.empty(N, dtype=np.int32)
    sorted_psw = np.empty(N, dtype=np.float32) if psw is not None else None
    U = lib().or_rle(N, _p(keys), _p(sorted_pos), _p(bags), _p(psw), _p(run_keys),
                     _p(run_offsets), _p(sorted_bag), _p(sorted_psw))
    return dict(U=int(U), run_keys=run_keys[:U].copy(), run_offsets=run_offsets[:U + 1].copy(),
                sorted_bag=sorted_bag, sorted_psw=sorted_psw)


def route(run_offsets, S=256, C=256):
    run_offsets = _c(run_offsets, np.int32)
    U = run_offsets.size - 1
    N = int(run_offsets[-1]) if U >= 0 else 0
    short_runs = np.empty(max(U, 1), dtype=np.int32)
    long_runs = np.empty(max(U, 1), dtype=np.int32)
    long_chunk_begin = np.empty(max(U, 1) + 1, dtype=np.int32)
    cap_chunks = N // C + U + 1
    chunk_run = np.empty(cap_chunks, dtype=np.int32)
    chunk_start = np.empty(cap_chunks, dtype=np.int32)
    counts = np.zeros(3, dtype=np.int64)
    _check(lib().or_route(U, _p(run_offsets), S, C, _p(short_runs), _p(long_runs),
                          _p(long_chunk_begin), _p(chunk_run), _p(chunk_start), _p(counts)))
    ns, nl, nc = (int(x) for x in counts)
    return dict(short_runs=short_runs[:ns].copy(), long_runs=long_runs[:nl].copy(),
                long_chunk_begin=long_chunk_begin[:nl + 1].copy(),
                chunk_run=chunk_run[:nc].copy(), chunk_start=chunk_start[:nc].copy())


def backward_adagrad(T, B, D, dtype, run_keys, run_offsets, sorted_bag, sorted_psw,
                     grad, W, m, lr, eps, wkeys=None, want_g=False):
    """Per run u: (g[u], w_new[u], m_new[u]) as unrounded doubles. W/m hold the
    rows of `wkeys` (sorted) or every stacked row when wkeys is None."""
    run_keys, run_offsets = _c(run_keys, np.int32), _c(run_offsets, np.int32)
    sorted_bag, sorted_psw = _c(sorted_bag, np.int32), _c(sorted_psw, np.float32)
    grad = _c(grad, np.float32)
    raw = _raw_weights(W, dtype)
    m = _c(m, np.float32)
    wk = _c(wkeys, np.int32)
    U = run_keys.size
    g = np.empty((U, D), dtype=np.float64) if want_g else None
    w_new = np.empty((U, D), dtype=np.float64)
    m_new = np.empty(U, dtype=np.float64)
    _check(lib().or_backward_adagrad(T, B, D, DTYPES[dtype], U, _p(run_keys), _p(run_offsets),
                                     _p(sorted_bag), _p(sorted_psw), _p(grad), _p(wk),
                                     0 if wk is None else wk.size, _p(raw), _p(m),
                                     float(lr), float(eps), _p(g), _p(w_new), _p(m_new)))
    return dict(g=g, w_new=w_new, m_new=m_new)


def histogram(T, B, E, rows, indices, offsets):
    rows, indices, offsets = _c(rows, np.int64), _c(indices, np.int32), _c(offsets, np.int32)
    H = np.empty(T * B * E, dtype=np.int32)
    _check(lib().or_histogram(T, B, E, _p(rows), _p(indices), _p(offsets), _p(H)))
    return H.reshape(T, B, E)


def preprocess(T, B, rows, indices, offsets, psw, S=256, C=256):
    """linearize + sort + rle + route, as one dict of metadata."""
    keys, bags = linearize(T, B, rows, indices, offsets)
    pos = sort(keys)
    r = rle(keys, pos, bags, psw)
    r.update(route(r["run_offsets"], S, C))
    r.update(keys=keys, bags=bags, sorted_pos=pos)
    return r
