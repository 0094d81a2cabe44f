"""Shared helpers of the GPU parity tests: run the library through its C ABI
on one batch, run the oracle on the same inputs, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from tests.helpers import TOL, rel_err
from workloads import init_state, init_weights, torch_dtype

META_INT = ["run_keys", "run_offsets", "sorted_pos", "sorted_bag", "short_runs", "long_runs",
            "long_chunk_begin", "chunk_run", "chunk_start"]


def lib():
    import bwd_tbe_pooled_amd as tbe
    return tbe


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """Host raw storage of a weight tensor: float32 values or uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def values_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def encode(vals: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of values exactly representable in dtype."""
    if dtype == "f32":
        return vals.astype(np.float32).view(np.uint32).astype(np.int64)
    if dtype == "f16":
        return vals.astype(np.float16).view(np.uint16).astype(np.int64)
    return (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)


def ulp_distance(bits_a: np.ndarray, bits_b: np.ndarray, dtype: str) -> np.ndarray:
    nb = 32 if dtype == "f32" else 16
    sign = np.int64(1) << (nb - 1)

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & sign, -(b & (sign - 1)), b)
    return np.abs(ordered(bits_a) - ordered(bits_b))


def device_batch(batch, device="cuda"):
    d = dict(indices=torch.from_numpy(batch.indices).to(device),
             offsets=torch.from_numpy(batch.offsets).to(device),
             psw=None if batch.psw is None else torch.from_numpy(batch.psw).to(device),
             grad=None if batch.grad is None else torch.from_numpy(batch.grad).to(device))
    return d


def make_desc(cfg, S=0, C=0, flags=0, timer=None, error_flags=None):
    tbe = lib()
    return tbe.Desc(cfg.T, cfg.D, cfg.B, cfg.rows, cfg.dtype, S, C, flags, timer,
                    error_flags=error_flags)


def run_library(cfg, batch, W, m, *, meta_in_forward: bool, backward_meta: bool = True,
                S=0, C=0, flags=0, dev=None, with_pos: bool = True, error_flags=None,
                timer=None):
    """Forward (+ preprocessing when meta_in_forward) and backward through the
    C ABI. W and m are updated in place. Returns out and the metadata."""
    tbe = lib()
    desc = make_desc(cfg, S, C, flags, timer=timer, error_flags=error_flags)
    dev = dev or device_batch(batch)
    N = batch.indices.size
    weighted = batch.psw is not None
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device="cuda")
    meta = tbe.Meta(desc, N, weighted, with_pos=with_pos)
    if meta_in_forward:
        ws = tbe.workspace(desc, N, weighted, tbe.TBE_OP_FORWARD_PREPROCESS)
        tbe.tbe_forward(desc, W, dev["indices"], dev["offsets"], dev["psw"], out, meta, ws)
    else:
        ws = tbe.workspace(desc, N, weighted, tbe.TBE_OP_FORWARD)
        tbe.tbe_forward(desc, W, dev["indices"], dev["offsets"], dev["psw"], out, None, ws)
        wsp = tbe.workspace(desc, N, weighted, tbe.TBE_OP_PREPROCESS)
        tbe.tbe_preprocess(desc, dev["indices"], dev["offsets"], dev["psw"], meta, wsp)
    op = tbe.TBE_OP_BACKWARD if backward_meta else tbe.TBE_OP_BACKWARD_SELF
    wsb = tbe.workspace(desc, N, weighted, op)
    tbe.tbe_backward_adagrad(desc, W, m, dev["grad"], dev["indices"], dev["offsets"], dev["psw"],
                             meta if backward_meta else None, cfg.lr, cfg.eps, wsb)
    torch.cuda.synchronize()
    return dict(out=out, meta=meta, path=tbe.tbe_select_path(desc, N, weighted))


def meta_host(meta, path):
    """Metadata trimmed to its device-side counts, as numpy."""
    counts = meta["counts"].cpu().numpy()
    if path == 1:
        return dict(counts=counts, hist=meta["hist"].cpu().numpy())
    U, ns, nl, nc = (int(x) for x in counts[:4])
    h = dict(counts=counts)
    h["run_keys"] = meta["run_keys"][:U].cpu().numpy()
    h["run_offsets"] = meta["run_offsets"][:U + 1].cpu().numpy()
    N = int(h["run_offsets"][-1])
    h["sorted_pos"] = meta["sorted_pos"][:N].cpu().numpy() if "sorted_pos" in meta.tensors else None
    h["sorted_bag"] = meta["sorted_bag"][:N].cpu().numpy()
    h["sorted_psw"] = meta["sorted_psw"][:N].cpu().numpy() if "sorted_psw" in meta.tensors else None
    h["short_runs"] = meta["short_runs"][:ns].cpu().numpy()
    h["long_runs"] = meta["long_runs"][:nl].cpu().numpy()
    h["long_chunk_begin"] = meta["long_chunk_begin"][:nl + 1].cpu().numpy()
    h["chunk_run"] = meta["chunk_run"][:nc].cpu().numpy()
    h["chunk_start"] = meta["chunk_start"][:nc].cpu().numpy()
    return h


def oracle_all(cfg, batch, W0_rows, m0_rows, wkeys, S=256, C=256):
    """The oracle on the whole batch; weights/state given for keys `wkeys`."""
    pre = oracle.preprocess(cfg.T, cfg.B, cfg.rows, batch.indices, batch.offsets, batch.psw, S, C)
    out = oracle.forward(cfg.T, cfg.B, cfg.D, cfg.dtype, batch.offsets, pre["keys"], batch.psw,
                         W0_rows, wkeys=wkeys)
    bw = oracle.backward_adagrad(cfg.T, cfg.B, cfg.D, cfg.dtype, pre["run_keys"],
                                 pre["run_offsets"], pre["sorted_bag"], pre["sorted_psw"],
                                 batch.grad, W0_rows, m0_rows, cfg.lr, cfg.eps, wkeys=wkeys)
    return pre, out, bw


def assert_meta_equal(h, pre):
    assert int(h["counts"][0]) == pre["U"]
    assert int(h["counts"][1]) == pre["short_runs"].size
    assert int(h["counts"][2]) == pre["long_runs"].size
    assert int(h["counts"][3]) == pre["chunk_run"].size
    for name in META_INT:
        if name == "sorted_pos" and h[name] is None:
            continue
        np.testing.assert_array_equal(h[name], pre[name], err_msg=name)
    if pre["sorted_psw"] is not None:
        np.testing.assert_array_equal(h["sorted_psw"].view(np.uint32),
                                      pre["sorted_psw"].view(np.uint32), err_msg="sorted_psw")


def assert_rows_match(cfg, W_after, m_after, keys, w_new, m_new, label=""):
    """Updated rows within the dtype's tolerance of the unrounded oracle values,
    within 1 ulp of the oracle rounded to storage; state within 1e-5."""
    if keys.size == 0:
        return 0.0, 0
    kt = torch.from_numpy(keys.astype(np.int64)).to(W_after.device)
    got = W_after.index_select(0, kt)
    got_vals = values_f64(got)
    err = rel_err(got_vals, w_new)
    assert err <= TOL[cfg.dtype], f"{label} weights rel err {err:.3g} > {TOL[cfg.dtype]}"
    ulps = ulp_distance(encode(got_vals.reshape(-1), cfg.dtype),
                        encode(oracle.round_to(w_new.reshape(-1), cfg.dtype), cfg.dtype), cfg.dtype)
    # Where the update cancels the weight almost exactly, the accumulator's
    # rounding can exceed one storage ulp of the tiny result; the relative
    # error above (floored at the row rms) covers those elements.
    w2 = w_new.reshape(w_new.shape[0], -1) if w_new.ndim > 1 else w_new.reshape(-1, 1)
    rms = np.sqrt(np.mean(w2 * w2, axis=1, keepdims=True))
    sizable = (np.abs(w2) >= rms / 16).reshape(-1)
    if sizable.any():
        assert ulps[sizable].max() <= 1, \
            f"{label} weights differ by {ulps[sizable].max()} ulp from the rounded oracle"
    gm = m_after.index_select(0, kt).cpu().numpy().astype(np.float64)
    merr = np.max(np.abs(gm - m_new) / np.maximum(np.abs(m_new), 1e-30)) if keys.size else 0.0
    assert merr <= 1e-5, f"{label} state rel err {merr:.3g}"
    return err, int(ulps.max()) if ulps.size else 0


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def assert_untouched_unchanged(W0, W_after, m0, m_after, touched_keys, chunk_rows=1 << 20):
    """Every row whose weights or state changed is a touched row."""
    touched = torch.zeros(W0.shape[0], dtype=torch.bool, device=W0.device)
    if touched_keys.size:
        touched[torch.from_numpy(touched_keys.astype(np.int64)).to(W0.device)] = True
    for a in range(0, W0.shape[0], chunk_rows):
        b = min(W0.shape[0], a + chunk_rows)
        changed = (_bits(W0[a:b]) != _bits(W_after[a:b])).any(dim=1)
        changed |= _bits(m0[a:b]) != _bits(m_after[a:b])
        bad = changed & ~touched[a:b]
        assert not bool(bad.any()), f"untouched rows changed, e.g. {int(bad.nonzero()[0]) + a}"


def fresh_params(cfg, m0="zeros"):
    W = init_weights(cfg, "cuda")
    m = init_state(cfg, "cuda", m0)
    return W, m


def host_rows(W, m, keys):
    kt = torch.from_numpy(keys.astype(np.int64)).to(W.device)
    return raw_bits(W.index_select(0, kt)), m.index_select(0, kt).cpu().numpy()


__all__ = ["run_library", "meta_host", "oracle_all", "assert_meta_equal", "assert_rows_match",
           "assert_untouched_unchanged", "fresh_params", "host_rows", "raw_bits", "values_f64",
           "device_batch", "make_desc", "torch_dtype", "rel_err", "TOL"]
