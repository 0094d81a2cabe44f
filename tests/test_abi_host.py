"""C ABI checks that need no GPU: the library loads, exports every function
include/tbe.h declares, validates arguments on the host before any launch, and
sizes metadata/workspace consistently. No compute call is made here."""
import ctypes
import json
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

tbe = pytest.importorskip("bwd_tbe_pooled_amd", reason="libtbe.so not built")


def _declared_functions():
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"\b(tbe_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_exports_every_declared_function():
    declared = _declared_functions()
    assert len(declared) >= 10
    lib = ctypes.CDLL(tbe.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in tbe.h but not exported"
    assert sorted(tbe.exported_symbols()) == declared


def _header_constants():
    """#define and enum constants of include/tbe.h: name -> integer value."""
    src = open(os.path.join(ROOT, "include", "tbe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    vals = {}
    for name, v in re.findall(r"#define\s+(TBE_[A-Z0-9_]+)\s+\(?(0x[0-9a-fA-F]+|\d+)u?\)?", src):
        vals[name] = int(v, 0)
    for name, v in re.findall(r"\b(TBE_[A-Z0-9_]+)\s*=\s*(0x[0-9a-fA-F]+|\d+)", src):
        vals[name] = int(v, 0)
    return vals


def test_binding_stages_and_flags_match_the_header():
    """The binding's stage names follow the header's TBE_STAGE_* order, and its
    flag and path constants have the header's values."""
    h = _header_constants()
    stages = sorted((v, k) for k, v in h.items() if k.startswith("TBE_STAGE_"))
    assert [v for v, _ in stages] == list(range(len(stages)))
    assert h["TBE_NUM_STAGES"] == len(stages) == tbe.TBE_NUM_STAGES == len(tbe.STAGES)
    assert [k[len("TBE_STAGE_"):].lower() for _, k in stages] == tbe.STAGES
    for name in ("TBE_FLAG_CHECK", "TBE_FLAG_VALIDATE", "TBE_FLAG_FUSED_LONG",
                 "TBE_FLAG_NO_HOT_ROWS", "TBE_FLAG_HOT_BACKWARD", "TBE_PATH_GENERIC",
                 "TBE_PATH_SMALL_TABLE"):
        assert getattr(tbe, name) == h[name], name


def test_status_strings():
    for s in range(6):
        assert tbe.tbe_status_str(s) and tbe.tbe_status_str(s) != "unknown status"
    assert tbe.tbe_status_str(99) == "unknown status"


def _desc(**kw):
    base = dict(T=2, D=16, B=8, rows=[100, 50], dtype="f32")
    base.update(kw)
    return tbe.Desc(**base)


def test_small_table_eligibility_follows_the_page():
    g = json.load(open(os.path.join(GOLDEN, "page1_thresholds.json")))["small_table"]
    T, B = 4, 32
    ok = dict(T=T, D=128, B=B, rows=[g["E_max"]] * T, dtype="f16")
    N_ok = g["L_min"] * T * B
    assert tbe.tbe_select_path(tbe.Desc(**ok), N_ok, False) == tbe.TBE_PATH_SMALL_TABLE
    # each violated condition falls back to the generic path
    cases = [
        (dict(ok, rows=[g["E_max"] + 1] + [g["E_max"]] * (T - 1)), N_ok, False),
        (dict(ok, D=g["D_min"] - 1), N_ok, False),
        (dict(ok, D=g["D_max"] + 1), N_ok, False),
        (ok, N_ok - 1, False),                                  # average L just below 64
        (dict(ok, dtype="bf16"), N_ok, False),
        (dict(ok, dtype="f32"), N_ok, False),
        (ok, N_ok, True),                                       # per-sample weights
        (dict(ok, flags=tbe.TBE_FLAG_FORCE_GENERIC), N_ok, False),
    ]
    for kw, N, w in cases:
        assert tbe.tbe_select_path(tbe.Desc(**kw), N, w) == tbe.TBE_PATH_GENERIC, (kw, N, w)
    assert tbe.tbe_select_path(tbe.Desc(**dict(ok, D=g["D_min"])), N_ok, False) == 1
    assert tbe.tbe_select_path(tbe.Desc(**dict(ok, rows=[1] * T)), N_ok, False) == 1


def test_bad_descriptions_are_rejected():
    assert tbe.tbe_select_path(_desc(), 10, False) == tbe.TBE_PATH_GENERIC
    assert tbe.tbe_select_path(_desc(flags=tbe.TBE_FLAG_FUSED_LONG), 10, False) == 0
    assert tbe.tbe_select_path(_desc(flags=tbe.TBE_FLAG_NO_HOT_ROWS), 10, False) == 0
    assert tbe.tbe_select_path(_desc(flags=tbe.TBE_FLAG_HOT_BACKWARD), 10, False) == 0
    for kw in [dict(T=0, rows=[]), dict(D=0), dict(B=-1), dict(rows=[100, 0]),
               dict(flags=0x40), dict(flags=0x80), dict(short_max=-1), dict(chunk=-3),
               dict(flags=tbe.TBE_FLAG_CHECK)]:   # the fused check needs an error word
        with pytest.raises(tbe.TbeError) as e:
            tbe.tbe_select_path(_desc(**kw), 10, False)
        assert e.value.status == tbe.TBE_ERR_ARG, kw
    # int32 limits (page 1, checklist item 6): sum of rows and N below 2^31
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_select_path(_desc(rows=[2 ** 30, 2 ** 30]), 10, False)
    assert e.value.status == tbe.TBE_ERR_UNSUPPORTED
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_select_path(_desc(), 2 ** 31, False)
    assert e.value.status == tbe.TBE_ERR_UNSUPPORTED
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_select_path(_desc(D=4099), 10, False)   # odd D beyond 4 passes of 64 lanes
    assert e.value.status == tbe.TBE_ERR_UNSUPPORTED


def test_meta_capacities_bound_the_run_structure():
    N = 100_000
    caps = dict(zip(tbe.META_FIELDS, tbe.tbe_meta_capacity(_desc(), N, True)))
    assert caps["counts"] == 8
    assert caps["run_keys"] == min(N, 150) and caps["run_offsets"] == caps["run_keys"] + 1
    assert caps["sorted_pos"] == caps["sorted_bag"] == caps["sorted_psw"] == N
    assert caps["long_runs"] == N // 256 and caps["long_chunk_begin"] == N // 256 + 1
    # sum of ceil(SL/C) over long runs <= N/C + number of long runs
    assert caps["chunk_run"] == caps["chunk_start"] == N // 256 + N // 256
    assert caps["hist"] == 0
    unw = dict(zip(tbe.META_FIELDS, tbe.tbe_meta_capacity(_desc(), N, False)))
    assert unw["sorted_psw"] == 0
    small = tbe.Desc(T=3, D=128, B=10, rows=[64] * 3, dtype="f16")
    sc = dict(zip(tbe.META_FIELDS, tbe.tbe_meta_capacity(small, 64 * 30, False)))
    assert sc["hist"] == 3 * 10 * 64 and sc["sorted_pos"] == 0


def test_workspace_sizes_grow_with_the_operation():
    d = _desc()
    N = 50_000
    f = tbe.tbe_workspace_bytes(d, N, False, tbe.TBE_OP_FORWARD)
    fp = tbe.tbe_workspace_bytes(d, N, False, tbe.TBE_OP_FORWARD_PREPROCESS)
    b = tbe.tbe_workspace_bytes(d, N, False, tbe.TBE_OP_BACKWARD)
    bs = tbe.tbe_workspace_bytes(d, N, False, tbe.TBE_OP_BACKWARD_SELF)
    assert 0 < f < fp and 0 < b < bs and fp < bs
    assert tbe.tbe_workspace_bytes(d, N, False, 17) == 0
    assert tbe.tbe_workspace_bytes(_desc(D=0), N, False, tbe.TBE_OP_FORWARD) == 0


def test_calls_reject_bad_arguments_before_any_launch():
    """Every error here is found on the host; no HIP call is reached (this
    container has no GPU, so a launch would fail with TBE_ERR_HIP instead)."""
    lib = tbe._lib
    d = _desc()
    fake = ctypes.c_void_p(256)      # never dereferenced on these paths
    ws_small = ctypes.c_void_p(4096)
    st = lib.tbe_forward(d.ref, fake, fake, fake, 10, None, fake, None, ws_small, 1, None)
    assert st == tbe.TBE_ERR_WORKSPACE
    st = lib.tbe_forward(d.ref, None, fake, fake, 10, None, fake, None, ws_small, 1 << 30, None)
    assert st == tbe.TBE_ERR_ARG
    st = lib.tbe_forward(None, fake, fake, fake, 10, None, fake, None, ws_small, 1 << 30, None)
    assert st == tbe.TBE_ERR_ARG
    bad = _desc(flags=0x100)
    st = lib.tbe_forward(bad.ref, fake, fake, fake, 10, None, fake, None, ws_small, 1 << 30, None)
    assert st == tbe.TBE_ERR_ARG
    # meta with missing arrays
    empty_meta = tbe.tbe_meta()
    st = lib.tbe_preprocess(d.ref, fake, fake, 10, None, ctypes.byref(empty_meta), ws_small,
                            1 << 30, None)
    assert st == tbe.TBE_ERR_ARG
    st = lib.tbe_backward_adagrad(d.ref, fake, None, fake, fake, fake, 10, None, None, 0.01,
                                  1e-8, ws_small, 1 << 30, None)
    assert st == tbe.TBE_ERR_ARG
    st = lib.tbe_backward_adagrad(d.ref, fake, fake, fake, fake, fake, 10, None, None, -1.0,
                                  1e-8, ws_small, 1 << 30, None)
    assert st == tbe.TBE_ERR_ARG
    # misaligned workspace
    st = lib.tbe_forward(d.ref, fake, fake, fake, 10, None, fake, None, ctypes.c_void_p(4100),
                         1 << 30, None)
    assert st == tbe.TBE_ERR_ARG


def test_int64_workspace_and_limits():
    """The int64 entry points take totals beyond int32 (page 1, checklist item
    6) but keep every table below 2^31 - 1 rows; only FORWARD and
    BACKWARD_SELF have an int64 form."""
    big = tbe.Desc(T=3, D=8, B=4096, rows=[1_200_000_000, 1_000_000_000, 500_000_000],
                   dtype="bf16")
    N = 3 * 4096 * 20
    assert tbe.tbe_workspace_bytes(big, N, True, tbe.TBE_OP_BACKWARD_SELF) == 0   # int32: no
    f = tbe.tbe_workspace_bytes_i64(big, N, True, tbe.TBE_OP_FORWARD)
    b = tbe.tbe_workspace_bytes_i64(big, N, True, tbe.TBE_OP_BACKWARD_SELF)
    assert 0 < f < b
    for op in (tbe.TBE_OP_FORWARD_PREPROCESS, tbe.TBE_OP_PREPROCESS, tbe.TBE_OP_BACKWARD):
        assert tbe.tbe_workspace_bytes_i64(big, N, True, op) == 0
    huge_table = tbe.Desc(T=1, D=8, B=16, rows=[2 ** 31 - 1], dtype="f32")
    assert tbe.tbe_workspace_bytes_i64(huge_table, 100, False, tbe.TBE_OP_FORWARD) == 0
    # N beyond int32: the int32 form refuses, the int64 form sizes one group's worth
    d = _desc()
    n_big = 3 * 2 ** 30
    assert tbe.tbe_workspace_bytes(d, n_big, False, tbe.TBE_OP_BACKWARD_SELF) == 0
    w_big = tbe.tbe_workspace_bytes_i64(d, n_big, False, tbe.TBE_OP_BACKWARD_SELF)
    w_cap = tbe.tbe_workspace_bytes_i64(d, 2 ** 31 - 2, False, tbe.TBE_OP_BACKWARD_SELF)
    assert w_big == w_cap > 0    # every part is bounded by what one group can hold
    # the int64 calls check their arguments on the host as well
    lib = tbe._lib
    fake = ctypes.c_void_p(256)
    st = lib.tbe_forward_i64(d.ref, fake, fake, fake, 10, None, fake, fake, 1, None)
    assert st == tbe.TBE_ERR_WORKSPACE
    st = lib.tbe_backward_adagrad_i64(d.ref, fake, None, fake, fake, fake, 10, None, 0.01, 1e-8,
                                      fake, 1 << 30, None)
    assert st == tbe.TBE_ERR_ARG
    with pytest.raises(TypeError):
        tbe.tbe_forward_i64(d, None, torch.zeros(4, dtype=torch.int32),
                            torch.zeros(3, dtype=torch.int64), None, None, None)


def test_int64_workspace_bounds_every_group():
    """The int64 workspace must hold the int32 workspace of any group of
    consecutive tables the call may form (any lookup count up to N), for
    each path and operation."""
    rng = np.random.default_rng(7)
    for case in range(300):
        T = int(rng.integers(1, 7))
        small = case % 3 == 0
        rows = [int(x) for x in (rng.integers(1, 65, T) if small else
                                 rng.integers(1, 2 ** int(rng.integers(4, 31)), T))]
        D = int(rng.choice([64, 96, 128])) if small else int(rng.integers(1, 257))
        B = int(rng.integers(1, 5000))
        dtype = "f16" if small else str(rng.choice(["f32", "f16", "bf16"]))
        weighted = bool(rng.integers(0, 2)) and not small
        N = int(rng.integers(0, 64 * T * B + 2))
        d = tbe.Desc(T=T, D=D, B=B, rows=rows, dtype=dtype)
        for op in (tbe.TBE_OP_FORWARD, tbe.TBE_OP_BACKWARD_SELF):
            total = tbe.tbe_workspace_bytes_i64(d, N, weighted, op)
            assert total > 0
            t0 = int(rng.integers(0, T))
            t1 = int(rng.integers(t0 + 1, T + 1))
            if sum(rows[t0:t1]) >= 2 ** 31 - 1:
                t1 = t0 + 1            # a group holds fewer than 2^31 - 1 rows
            sub = tbe.Desc(T=t1 - t0, D=D, B=B, rows=rows[t0:t1], dtype=dtype)
            for Ng in (0, N, int(rng.integers(0, N + 1))):
                need = tbe.tbe_workspace_bytes(sub, Ng, weighted, op)
                assert 0 < need <= total, (case, T, rows, D, B, N, Ng, t0, t1, op)


def test_build_script_runs_without_the_library():
    """A clean checkout has no libtbe.so, and importing the package refuses to
    run without it; the build entry point must therefore load the build
    script without importing the package."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import importlib.util, os, sys\n"
        f"root = {root!r}\n"
        "spec = importlib.util.spec_from_file_location('b', os.path.join(root, 'bwd_tbe_pooled_amd', 'build.py'))\n"
        "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
        "assert callable(m.build) and 'bwd_tbe_pooled_amd' not in sys.modules\n"
        "src = open(os.path.join(root, '__graft_entry__.py')).read()\n"
        "body = src.split('def build()')[1].split('def ')[0]\n"
        "assert 'spec_from_file_location' in body\n"
        "assert body.index('hipbuild.build()') < body.index('import bwd_tbe_pooled_amd')\n"
    )
    env = dict(os.environ, TBE_LIBRARY=os.path.join(root, "no_such_libtbe.so"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_noalloc_refuses_beyond_its_scratch_before_any_work():
    """The backward without allocation checks the problem's scratch against
    its built-in array on the host, before any HIP call."""
    lib = tbe._lib
    d = _desc(T=2, D=128, B=8, rows=[1000, 1000], dtype="f16")
    N = 40_000_000
    assert tbe.tbe_workspace_bytes(d, N, False, tbe.TBE_OP_BACKWARD) > tbe.TBE_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)
    meta = tbe.tbe_meta()
    st = lib.tbe_backward_adagrad_noalloc(d.ref, fake, fake, fake, fake, fake, N, None,
                                          ctypes.byref(meta), 0.01, 1e-8, None)
    assert st == tbe.TBE_ERR_WORKSPACE
    assert b"scratch" in lib.tbe_last_error()
    # a missing metadata argument is an argument error
    st = lib.tbe_backward_adagrad_noalloc(d.ref, fake, fake, fake, fake, fake, 10, None, None,
                                          0.01, 1e-8, None)
    assert st == tbe.TBE_ERR_ARG


def test_binding_rejects_host_tensors():
    """The wrappers pass raw device pointers: a host tensor is refused before
    any call."""
    d = _desc(T=2, D=16, B=4, rows=[100, 50], dtype="f32")
    idx = torch.zeros(8, dtype=torch.int32)
    off = torch.arange(0, 9, dtype=torch.int32)
    W = torch.zeros((150, 16), dtype=torch.float32)
    out = torch.zeros((4, 32), dtype=torch.float32)
    with pytest.raises(TypeError, match="device"):
        tbe.tbe_forward(d, W, idx, off, None, out, None, torch.zeros(1024, dtype=torch.uint8))
