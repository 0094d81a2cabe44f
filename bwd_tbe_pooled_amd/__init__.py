"""Python binding of the MI355X table-batched embedding library (libtbe.so).

Argument marshalling only: every step of the forward, the transpose (sort +
run-length encoding + routing) and the backward with row-wise Adagrad runs in
the library's HIP kernels. The functions carry the C ABI's names
(include/tbe.h) and take torch tensors, passing their device pointers and the
current HIP stream. There is no CPU fallback: importing this package fails if
the library has not been built (python bwd_tbe_pooled_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# TBE_LIBRARY may name another build of the same library (development builds).
LIB_PATH = os.environ.get("TBE_LIBRARY") or os.path.join(_HERE, "libtbe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python bwd_tbe_pooled_amd/build.py`")

# torch first: the library then binds to the HIP runtime torch has loaded,
# so tensors, streams and kernels share one runtime in the process (loading
# the library first would bring in a second HIP runtime beside torch's).
import torch  # noqa: E402

_lib = ctypes.CDLL(LIB_PATH)

# --- C types ----------------------------------------------------------------
TBE_OK, TBE_ERR_ARG, TBE_ERR_UNSUPPORTED, TBE_ERR_WORKSPACE, TBE_ERR_INDEX_RANGE, TBE_ERR_HIP = range(6)
TBE_F32, TBE_F16, TBE_BF16 = 0, 1, 2
TBE_FLAG_VALIDATE, TBE_FLAG_FORCE_GENERIC, TBE_FLAG_CHECK, TBE_FLAG_FUSED_LONG = 0x1, 0x2, 0x4, 0x8
TBE_FLAG_NO_HOT_ROWS, TBE_FLAG_HOT_BACKWARD = 0x10, 0x20
TBE_ERROR_INDEX = 0x1
TBE_PATH_GENERIC, TBE_PATH_SMALL_TABLE = 0, 1
(TBE_OP_FORWARD, TBE_OP_FORWARD_PREPROCESS, TBE_OP_PREPROCESS, TBE_OP_BACKWARD,
 TBE_OP_BACKWARD_SELF) = range(5)
STAGES = ["fwd_pool", "linearize", "sort", "rle_route", "bwd_short", "bwd_long", "bwd_apply",
          "small_fwd", "small_bwd", "small_apply", "validate", "long_schedule", "small_count",
          "bwd_hot", "hot_plan", "bwd_hot_plan"]
TBE_NUM_STAGES = len(STAGES)
TBE_NOALLOC_SCRATCH_BYTES = 64 << 20   # built-in scratch of tbe_backward_adagrad_noalloc
META_FIELDS = ["counts", "run_keys", "run_offsets", "sorted_pos", "sorted_bag", "sorted_psw",
               "short_runs", "long_runs", "long_chunk_begin", "chunk_run", "chunk_start", "hist"]
TBE_META_NUM_ARRAYS = len(META_FIELDS)
DTYPE_CODES = {"f32": TBE_F32, "f16": TBE_F16, "bf16": TBE_BF16}


class tbe_desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("B", ctypes.c_int32),
                ("rows", ctypes.POINTER(ctypes.c_int64)), ("wdtype", ctypes.c_int),
                ("short_max", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("timer", ctypes.c_void_p),
                ("error_flags", ctypes.c_void_p)]


class tbe_meta(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in META_FIELDS]


_P = ctypes.c_void_p
_lib.tbe_status_str.restype = ctypes.c_char_p
_lib.tbe_status_str.argtypes = [ctypes.c_int]
_lib.tbe_select_path.restype = ctypes.c_int32
_lib.tbe_select_path.argtypes = [ctypes.POINTER(tbe_desc), ctypes.c_int64, ctypes.c_int32]
_lib.tbe_meta_capacity.restype = ctypes.c_int
_lib.tbe_meta_capacity.argtypes = [ctypes.POINTER(tbe_desc), ctypes.c_int64, ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_int64)]
_lib.tbe_workspace_bytes.restype = ctypes.c_size_t
_lib.tbe_workspace_bytes.argtypes = [ctypes.POINTER(tbe_desc), ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_int]
_lib.tbe_forward.restype = ctypes.c_int
_lib.tbe_forward.argtypes = [ctypes.POINTER(tbe_desc), _P, _P, _P, ctypes.c_int64, _P, _P,
                             ctypes.POINTER(tbe_meta), _P, ctypes.c_size_t, _P]
_lib.tbe_preprocess.restype = ctypes.c_int
_lib.tbe_preprocess.argtypes = [ctypes.POINTER(tbe_desc), _P, _P, ctypes.c_int64, _P,
                                ctypes.POINTER(tbe_meta), _P, ctypes.c_size_t, _P]
_lib.tbe_backward_adagrad.restype = ctypes.c_int
_lib.tbe_backward_adagrad.argtypes = [ctypes.POINTER(tbe_desc), _P, _P, _P, _P, _P,
                                      ctypes.c_int64, _P, ctypes.POINTER(tbe_meta),
                                      ctypes.c_double, ctypes.c_double, _P, ctypes.c_size_t, _P]
_lib.tbe_workspace_bytes_i64.restype = ctypes.c_size_t
_lib.tbe_workspace_bytes_i64.argtypes = [ctypes.POINTER(tbe_desc), ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int]
_lib.tbe_forward_i64.restype = ctypes.c_int
_lib.tbe_forward_i64.argtypes = [ctypes.POINTER(tbe_desc), _P, _P, _P, ctypes.c_int64, _P, _P,
                                 _P, ctypes.c_size_t, _P]
_lib.tbe_backward_adagrad_i64.restype = ctypes.c_int
_lib.tbe_backward_adagrad_i64.argtypes = [ctypes.POINTER(tbe_desc), _P, _P, _P, _P, _P,
                                          ctypes.c_int64, _P, ctypes.c_double, ctypes.c_double,
                                          _P, ctypes.c_size_t, _P]
_lib.tbe_backward_adagrad_noalloc.restype = ctypes.c_int
_lib.tbe_backward_adagrad_noalloc.argtypes = [ctypes.POINTER(tbe_desc), _P, _P, _P, _P, _P,
                                              ctypes.c_int64, _P, ctypes.POINTER(tbe_meta),
                                              ctypes.c_double, ctypes.c_double, _P]
_lib.tbe_probe_row_gather.restype = ctypes.c_int
_lib.tbe_probe_row_gather.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_int64, _P, _P]
TBE_PROBE_SINK_FLOATS = 16384
_lib.tbe_timer_create.restype = ctypes.c_int
_lib.tbe_timer_create.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
_lib.tbe_timer_reset.restype = ctypes.c_int
_lib.tbe_timer_reset.argtypes = [_P]
_lib.tbe_timer_read.restype = ctypes.c_int
_lib.tbe_timer_read.argtypes = [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
_lib.tbe_timer_destroy.restype = None
_lib.tbe_timer_destroy.argtypes = [_P]


_lib.tbe_last_error.restype = ctypes.c_char_p
_lib.tbe_last_error.argtypes = []


class TbeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {tbe_status_str(status)} (status {status})"
        if status == TBE_ERR_HIP:
            msg += ": " + _lib.tbe_last_error().decode()
        super().__init__(msg)


def tbe_status_str(status: int) -> str:
    return _lib.tbe_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != TBE_OK:
        raise TbeError(status, where)


# --- description ----------------------------------------------------------------
class Desc:
    """Owns a tbe_desc and the host rows array it points to."""

    def __init__(self, T: int, D: int, B: int, rows: Sequence[int], dtype: str,
                 short_max: int = 0, chunk: int = 0, flags: int = 0, timer: "Timer" = None,
                 error_flags=None):
        self._rows = (ctypes.c_int64 * len(rows))(*[int(r) for r in rows])
        self.c = tbe_desc(T=int(T), D=int(D), B=int(B),
                          rows=ctypes.cast(self._rows, ctypes.POINTER(ctypes.c_int64)),
                          wdtype=DTYPE_CODES[dtype], short_max=int(short_max), chunk=int(chunk),
                          flags=int(flags), timer=timer.handle if timer else None,
                          error_flags=_ptr(error_flags))
        self._error_flags = error_flags  # keeps the device word alive
        self.T, self.D, self.B, self.dtype = int(T), int(D), int(B), dtype
        self.rows = [int(r) for r in rows]

    def set_timer(self, timer: Optional["Timer"]):
        self.c.timer = timer.handle if timer else None

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_TORCH_W = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _need(t, name, dtype, numel=None, shape=None):
    """Raise TypeError unless `t` is a contiguous device tensor of `dtype`
    (and `numel` elements / `shape`): the library reads raw device memory, so
    a host tensor, an int64 array passed as int32 or a strided view would be
    read as something else."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise TypeError(f"{name}: must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name}: must be contiguous")
    if numel is not None and t.numel() != numel:
        raise TypeError(f"{name}: expected {numel} elements, got {t.numel()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise TypeError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_args(desc: "Desc", idx_dtype, W=None, indices=None, offsets=None, psw=None, out=None,
                grad_out=None, momentum=None):
    _need(indices, "indices", idx_dtype)
    N = indices.numel() if indices is not None else None
    _need(offsets, "offsets", idx_dtype, numel=desc.T * desc.B + 1)
    _need(psw, "psw", torch.float32, numel=N)
    _need(W, "W", _TORCH_W[desc.dtype], numel=sum(desc.rows) * desc.D)
    _need(momentum, "momentum", torch.float32, numel=sum(desc.rows))
    _need(out, "out", torch.float32, shape=(desc.B, desc.T * desc.D))
    _need(grad_out, "grad_out", torch.float32, shape=(desc.B, desc.T * desc.D))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def tbe_select_path(desc: Desc, N: int, weighted: bool) -> int:
    r = _lib.tbe_select_path(desc.ref, int(N), int(bool(weighted)))
    if r < 0:
        raise TbeError(-r, "tbe_select_path")
    return r


def tbe_meta_capacity(desc: Desc, N: int, weighted: bool) -> list:
    caps = (ctypes.c_int64 * TBE_META_NUM_ARRAYS)()
    _check(_lib.tbe_meta_capacity(desc.ref, int(N), int(bool(weighted)), caps), "tbe_meta_capacity")
    return list(caps)


def tbe_workspace_bytes(desc: Desc, N: int, weighted: bool, op: int) -> int:
    return int(_lib.tbe_workspace_bytes(desc.ref, int(N), int(bool(weighted)), int(op)))


class Meta:
    """Device buffers of a tbe_meta, allocated to the library's capacities."""

    def __init__(self, desc: Desc, N: int, weighted: bool, device="cuda", with_pos: bool = True):
        """with_pos=False leaves sorted_pos NULL: the sort then does not carry
        lookup positions (the backward never reads them)."""
        caps = tbe_meta_capacity(desc, N, weighted)
        self.caps = dict(zip(META_FIELDS, caps))
        self.path = tbe_select_path(desc, N, weighted)
        if self.path == TBE_PATH_SMALL_TABLE:
            used = {"counts", "hist"}
        else:
            used = set(META_FIELDS) - {"hist"} - (set() if weighted else {"sorted_psw"})
            if not with_pos:
                used -= {"sorted_pos"}
        self.tensors = {}
        for name in META_FIELDS:
            if name not in used:
                continue
            dt = torch.uint8 if name == "hist" else (torch.float32 if name == "sorted_psw" else torch.int32)
            # at least one element, so that every array the path uses is non-null
            self.tensors[name] = torch.empty(max(int(self.caps[name]), 1), dtype=dt, device=device)
        self.c = tbe_meta(**{n: (t.data_ptr() if t is not None else None)
                             for n, t in ((n, self.tensors.get(n)) for n in META_FIELDS)})

    def __getitem__(self, name):
        return self.tensors[name]

    @property
    def ref(self):
        return ctypes.byref(self.c)


def workspace(desc: Desc, N: int, weighted: bool, op: int, device="cuda"):
    nbytes = tbe_workspace_bytes(desc, N, weighted, op)
    if nbytes == 0:
        raise TbeError(TBE_ERR_ARG, "tbe_workspace_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# --- the three calls ------------------------------------------------------------
def tbe_forward(desc: Desc, W, indices, offsets, psw, out, meta: Optional[Meta], ws, stream=None):
    _check_args(desc, torch.int32, W=W, indices=indices, offsets=offsets, psw=psw, out=out)
    N = indices.numel()
    _check(_lib.tbe_forward(desc.ref, _ptr(W), _ptr(indices), _ptr(offsets), N, _ptr(psw),
                            _ptr(out), meta.ref if meta is not None else None, _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)), "tbe_forward")


def tbe_preprocess(desc: Desc, indices, offsets, psw, meta: Meta, ws, stream=None):
    _check_args(desc, torch.int32, indices=indices, offsets=offsets, psw=psw)
    N = indices.numel()
    _check(_lib.tbe_preprocess(desc.ref, _ptr(indices), _ptr(offsets), N, _ptr(psw), meta.ref,
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "tbe_preprocess")


def tbe_backward_adagrad(desc: Desc, W, momentum, grad_out, indices, offsets, psw,
                         meta: Optional[Meta], lr: float, eps: float, ws, stream=None):
    _check_args(desc, torch.int32, W=W, indices=indices, offsets=offsets, psw=psw,
                grad_out=grad_out, momentum=momentum)
    N = indices.numel()
    _check(_lib.tbe_backward_adagrad(desc.ref, _ptr(W), _ptr(momentum), _ptr(grad_out),
                                     _ptr(indices), _ptr(offsets), N, _ptr(psw),
                                     meta.ref if meta is not None else None, float(lr),
                                     float(eps), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "tbe_backward_adagrad")


def tbe_backward_adagrad_noalloc(desc: Desc, W, momentum, grad_out, indices, offsets, psw,
                                 meta: Meta, lr: float, eps: float, stream=None):
    """tbe_backward_adagrad with metadata and no workspace: the library's
    built-in per-device scratch (TBE_NOALLOC_SCRATCH_BYTES) serves instead.
    Calls on one device must not overlap."""
    _check_args(desc, torch.int32, W=W, indices=indices, offsets=offsets, psw=psw,
                grad_out=grad_out, momentum=momentum)
    N = indices.numel()
    _check(_lib.tbe_backward_adagrad_noalloc(desc.ref, _ptr(W), _ptr(momentum), _ptr(grad_out),
                                             _ptr(indices), _ptr(offsets), N, _ptr(psw),
                                             meta.ref if meta is not None else None, float(lr),
                                             float(eps), _stream(stream)),
           "tbe_backward_adagrad_noalloc")


# --- int64 indices and offsets ----------------------------------------------------
def tbe_workspace_bytes_i64(desc: Desc, N: int, weighted: bool, op: int) -> int:
    return int(_lib.tbe_workspace_bytes_i64(desc.ref, int(N), int(bool(weighted)), int(op)))


def workspace_i64(desc: Desc, N: int, weighted: bool, op: int, device="cuda"):
    nbytes = tbe_workspace_bytes_i64(desc, N, weighted, op)
    if nbytes == 0:
        raise TbeError(TBE_ERR_ARG, "tbe_workspace_bytes_i64")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _need_i64(*tensors):
    for t in tensors:
        if t is not None and t.dtype != torch.int64:
            raise TypeError(f"the _i64 entry points take int64 indices and offsets, got {t.dtype}")


def tbe_forward_i64(desc: Desc, W, indices, offsets, psw, out, ws, stream=None):
    _need_i64(indices, offsets)
    _check_args(desc, torch.int64, W=W, indices=indices, offsets=offsets, psw=psw, out=out)
    N = indices.numel()
    _check(_lib.tbe_forward_i64(desc.ref, _ptr(W), _ptr(indices), _ptr(offsets), N, _ptr(psw),
                                _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "tbe_forward_i64")


def tbe_backward_adagrad_i64(desc: Desc, W, momentum, grad_out, indices, offsets, psw,
                             lr: float, eps: float, ws, stream=None):
    _need_i64(indices, offsets)
    _check_args(desc, torch.int64, W=W, indices=indices, offsets=offsets, psw=psw,
                grad_out=grad_out, momentum=momentum)
    N = indices.numel()
    _check(_lib.tbe_backward_adagrad_i64(desc.ref, _ptr(W), _ptr(momentum), _ptr(grad_out),
                                         _ptr(indices), _ptr(offsets), N, _ptr(psw), float(lr),
                                         float(eps), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)), "tbe_backward_adagrad_i64")


# --- measurement aid (include/tbe_probe.h) ---------------------------------------------
def tbe_probe_row_gather(src, rows, sink, stream=None):
    """Gather rows[i] of the float32 matrix src [R, F] (F = 64, 128 or 256)
    with the library's load shape; one float per wave to sink."""
    _need(src, "src", torch.float32)
    _need(rows, "rows", torch.int32)
    _need(sink, "sink", torch.float32, numel=TBE_PROBE_SINK_FLOATS)
    if src.dim() != 2:
        raise TypeError("src: expected a [rows, floats] matrix")
    _check(_lib.tbe_probe_row_gather(_ptr(src), src.shape[0], src.shape[1], _ptr(rows),
                                     rows.numel(), _ptr(sink), _stream(stream)),
           "tbe_probe_row_gather")


# --- stage timer -----------------------------------------------------------------
class Timer:
    def __init__(self, capacity: int = 256):
        h = ctypes.c_void_p()
        _check(_lib.tbe_timer_create(int(capacity), ctypes.byref(h)), "tbe_timer_create")
        self.handle = h
        # kept on the instance: at interpreter exit the module's globals may
        # already be gone when the timer is collected
        self._destroy = _lib.tbe_timer_destroy

    def reset(self):
        _check(_lib.tbe_timer_reset(self.handle), "tbe_timer_reset")

    def read(self) -> dict:
        ms = (ctypes.c_float * TBE_NUM_STAGES)()
        n = (ctypes.c_int32 * TBE_NUM_STAGES)()
        _check(_lib.tbe_timer_read(self.handle, ms, n), "tbe_timer_read")
        return {STAGES[i]: (float(ms[i]), int(n[i])) for i in range(TBE_NUM_STAGES)}

    def __del__(self):
        h = getattr(self, "handle", None)
        destroy = getattr(self, "_destroy", None)
        if h and destroy is not None:
            destroy(h)
            self.handle = None


def exported_symbols() -> list:
    """Names the library exports from include/tbe.h (used by host tests)."""
    return ["tbe_status_str", "tbe_last_error", "tbe_select_path", "tbe_meta_capacity", "tbe_workspace_bytes",
            "tbe_forward", "tbe_preprocess", "tbe_backward_adagrad", "tbe_workspace_bytes_i64",
            "tbe_forward_i64", "tbe_backward_adagrad_i64", "tbe_backward_adagrad_noalloc",
            "tbe_probe_row_gather", "tbe_timer_create",
            "tbe_timer_reset", "tbe_timer_read", "tbe_timer_destroy"]
