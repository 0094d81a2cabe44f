"""The backward that allocates nothing (tbe_backward_adagrad_noalloc) against
tbe_backward_adagrad with a caller workspace: the same metadata, weights,
state and upstream gradient must give the same updated weights and state, bit
for bit (the two run the same kernels). Two calls in a row on each path, the
second on a smaller batch, so the second runs on scratch the first left
behind; the same with the hot rows' contraction on; plus the refusal of a
problem whose scratch would not fit."""
import numpy as np
import pytest
import torch

from tests.gpu_common import device_batch, fresh_params, make_desc
from workloads import DEMO3, LARGE, MEDIUM, SMALL_TABLE, make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _step_pair(cfg, B, flags=0, timer=None):
    """Forward with metadata, then the backward through both entry points on
    copies of the same weights and state."""
    import bwd_tbe_pooled_amd as tbe
    batch = make_batch(cfg, B=B)
    c = batch.cfg
    dev = device_batch(batch)
    N = batch.indices.size
    weighted = batch.psw is not None
    desc = make_desc(c, flags=flags, timer=timer)
    need = tbe.tbe_workspace_bytes(desc, N, weighted, tbe.TBE_OP_BACKWARD)
    assert 0 < need <= tbe.TBE_NOALLOC_SCRATCH_BYTES, (c.name, B, need)
    W, m = fresh_params(c, m0="uniform")
    out = torch.empty((c.B, c.T * c.D), dtype=torch.float32, device="cuda")
    meta = tbe.Meta(desc, N, weighted)
    tbe.tbe_forward(desc, W, dev["indices"], dev["offsets"], dev["psw"], out, meta,
                    tbe.workspace(desc, N, weighted, tbe.TBE_OP_FORWARD_PREPROCESS))
    W1, m1, W2, m2 = W.clone(), m.clone(), W.clone(), m.clone()
    tbe.tbe_backward_adagrad(desc, W1, m1, dev["grad"], dev["indices"], dev["offsets"], dev["psw"],
                             meta, c.lr, c.eps, tbe.workspace(desc, N, weighted, tbe.TBE_OP_BACKWARD))
    tbe.tbe_backward_adagrad_noalloc(desc, W2, m2, dev["grad"], dev["indices"], dev["offsets"],
                                     dev["psw"], meta, c.lr, c.eps)
    torch.cuda.synchronize()
    assert not torch.equal(_bits(W1), _bits(W)), "the step changed nothing"
    assert torch.equal(_bits(W1), _bits(W2)), f"{c.name} B={B}: weights differ"
    assert torch.equal(_bits(m1), _bits(m2)), f"{c.name} B={B}: state differs"
    return N


@pytest.mark.parametrize("cfg,B1,B2", [
    (MEDIUM, 4096, 1024),        # f16 weights, f32 partials, long runs
    (DEMO3, 4096, 700),          # f32 weights, f64 partials
    (SMALL_TABLE, 2048, 300),    # small-table path, split partials
], ids=["f16_generic", "f32_generic", "small_table"])
def test_noalloc_matches_workspace_call_twice(cfg, B1, B2):
    print(f"\n[noalloc] {cfg.name} B={B1} then B={B2}", flush=True)
    n1 = _step_pair(cfg, B1)
    n2 = _step_pair(cfg, B2)
    assert n2 < n1


def test_noalloc_fused_long_matches():
    import bwd_tbe_pooled_amd as tbe
    print("\n[noalloc] fused long path", flush=True)
    _step_pair(MEDIUM, 2048, flags=tbe.TBE_FLAG_FUSED_LONG)


@pytest.mark.parametrize("cfg,B1,B2", [
    (MEDIUM, 4096, 1024),        # f16 weights, unweighted
    (LARGE, 2048, 1024),         # the benchmark's tables: bf16, weighted
], ids=["f16_unweighted", "bf16_weighted"])
def test_noalloc_hot_backward_matches(cfg, B1, B2):
    """The hot rows' contraction (TBE_FLAG_HOT_BACKWARD, the benchmark's
    configuration): its plan, segment partials and flags come from the
    scratch too."""
    import bwd_tbe_pooled_amd as tbe
    print(f"\n[noalloc] hot rows' backward, {cfg.name} B={B1} then B={B2}", flush=True)
    for B in (B1, B2):
        timer = tbe.Timer(4)
        _step_pair(cfg, B, flags=tbe.TBE_FLAG_HOT_BACKWARD, timer=timer)
        assert timer.read()["bwd_hot"][1] == 2, "the contraction did not run in both calls"


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    import bwd_tbe_pooled_amd as tbe
    cfg = MEDIUM
    N = 40_000_000       # about 2 x N/128 chunk partials of 512 bytes: beyond 64 MiB
    desc = make_desc(cfg)
    assert tbe.tbe_workspace_bytes(desc, N, False, tbe.TBE_OP_BACKWARD) > tbe.TBE_NOALLOC_SCRATCH_BYTES
    W, m = fresh_params(cfg)
    W0 = W.clone()
    idx = torch.zeros(N, dtype=torch.int32, device="cuda")
    off = torch.zeros(cfg.T * cfg.B + 1, dtype=torch.int32, device="cuda")
    grad = torch.zeros((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device="cuda")
    meta = tbe.Meta(desc, 1, False)     # never read: the call stops before any work
    with pytest.raises(tbe.TbeError) as e:
        tbe.tbe_backward_adagrad_noalloc(desc, W, m, grad, idx, off, None, meta, cfg.lr, cfg.eps)
    assert e.value.status == tbe.TBE_ERR_WORKSPACE
    assert "scratch" in tbe._lib.tbe_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(_bits(W), _bits(W0))
