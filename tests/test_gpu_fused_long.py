"""The single-launch long-run path (TBE_FLAG_FUSED_LONG): each chunk publishes
its partial with a device-scope release and counts itself in on its run; the
last chunk to arrive reduces the run's partials in chunk order and applies
Adagrad (page 1, backward section, the fused path of figure 3).

Ordering and race checks: the fused path (which takes no hot-row path) must
give the same bits as the two launches (chunk partials, then a separate
apply) under TBE_FLAG_NO_HOT_ROWS, which reduce in the same order. A reader that saw a partial before it was complete would
break that:
- the backward workspace is filled with 0xFF bytes first, so a partial read
  before its chunk wrote it is a NaN;
- two backward steps with different upstream gradients reuse one workspace,
  so a partial left from the first step is a wrong value in the second;
- small chunk lengths put hundreds of chunks on one run, all counting in on
  one counter.
Parity with the oracle itself is in the parity tests (the same cases run
with this flag)."""
import numpy as np
import pytest
import torch

from tests.gpu_common import device_batch, fresh_params, lib, make_desc
from workloads import WORKLOADS, make_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_tbe_pooled_amd  # noqa: F401  (fails loudly if the library is missing)


def _steps(cfg, batch, dev, grads, flags, S, C):
    """Preprocess once, then one backward per gradient, all on one workspace."""
    tbe = lib()
    desc = make_desc(cfg, S, C, flags)
    N = batch.indices.size
    weighted = batch.psw is not None
    W, m = fresh_params(cfg)
    meta = tbe.Meta(desc, N, weighted, with_pos=False)
    wsp = tbe.workspace(desc, N, weighted, tbe.TBE_OP_PREPROCESS)
    tbe.tbe_preprocess(desc, dev["indices"], dev["offsets"], dev["psw"], meta, wsp)
    del wsp
    wsb = tbe.workspace(desc, N, weighted, tbe.TBE_OP_BACKWARD)
    wsb.fill_(255)  # an unwritten partial reads as NaN
    for g in grads:
        tbe.tbe_backward_adagrad(desc, W, m, g, dev["indices"], dev["offsets"], dev["psw"], meta,
                                 cfg.lr, cfg.eps, wsb)
    torch.cuda.synchronize()
    counts = meta["counts"].cpu().numpy()
    return W, m, counts


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _compare(name, B, S, C):
    cfg = WORKLOADS[name]
    batch = make_batch(cfg, B=B)
    cfg = batch.cfg
    print(f"\n[fused-long] {cfg.name} T={cfg.T} B={cfg.B} D={cfg.D} {cfg.dtype} "
          f"N={batch.indices.size} S={S or 256} C={C or 256}", flush=True)
    dev = device_batch(batch)
    gen = torch.Generator(device="cuda").manual_seed(7)
    g2 = torch.randn(dev["grad"].shape, generator=gen, device="cuda", dtype=torch.float32)
    grads = [dev["grad"], g2]
    tbe = lib()
    W0, m0, c0 = _steps(cfg, batch, dev, grads, tbe.TBE_FLAG_NO_HOT_ROWS, S, C)
    W1, m1, c1 = _steps(cfg, batch, dev, grads, tbe.TBE_FLAG_FUSED_LONG, S, C)
    np.testing.assert_array_equal(c0, c1)
    n_long, n_chunks = int(c1[2]), int(c1[3])
    print(f"[fused-long] long runs {n_long}, chunks {n_chunks}", flush=True)
    assert n_long > 0 and n_chunks > n_long
    assert not bool(torch.isnan(W1.float()).any())
    assert torch.equal(_bits(W0), _bits(W1)), "weights differ from the two-launch path"
    assert torch.equal(_bits(m0), _bits(m1)), "state differs from the two-launch path"


@pytest.mark.parametrize("name,B,S,C", [
    ("demo3_d16_f32_b4k", None, 4, 3),         # f32 weights: f64 partials; many chunks per run
    ("t16_e1m_d128_f16_b16k", None, 0, 0),     # default S = C = 256
    ("t16_e1m_d128_f16_b16k", 4096, 16, 16),   # hundreds of chunks on the hottest runs
    ("t32_e2m_d128_bf16_b128k", 8192, 0, 0),   # weighted bf16
])
def test_fused_long_matches_two_launches_bitwise(name, B, S, C):
    _compare(name, B, S, C)


@pytest.mark.slow
def test_fused_long_full_size_matches_two_launches_bitwise():
    """T=32, E=2M, D=128 bf16, B=131072 weighted: about 288K chunks."""
    _compare("t32_e2m_d128_bf16_b128k", None, 0, 0)
