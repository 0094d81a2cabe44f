"""The step captured in a HIP graph. The library enqueues only kernels on the
caller's stream (no host synchronisation, no memset nodes, no allocation), so
a forward with preprocessing plus a backward can be captured once and
replayed. Each replay starts from the same weights and state, restored by
eager copies with a synchronisation in between, and must give the eager
step's bits."""
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


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("name,B,hot", [("t16_e1m_d128_f16_b16k", 2048, False),
                                        ("t32_e2m_d128_bf16_b128k", 1024, False),
                                        ("t32_e2m_d128_bf16_b128k", 1024, True),
                                        ("small_t64_e64_d128_f16_b32k", 512, False)],
                         ids=["f16", "bf16_weighted", "bf16_weighted_hot_backward", "small_table"])
def test_step_replayed_from_a_graph_matches_eager(name, B, hot):
    """With hot: the benchmark's configuration (TBE_FLAG_HOT_BACKWARD), whose
    hot-row plan and contraction run inside the captured backward."""
    tbe = lib()
    batch = make_batch(WORKLOADS[name], B=B)
    cfg = batch.cfg
    print(f"\n[graph] {cfg.name} B={cfg.B} N={batch.indices.size} hot={hot}", flush=True)
    dev = device_batch(batch)
    N = batch.indices.size
    weighted = dev["psw"] is not None
    desc = make_desc(cfg, flags=tbe.TBE_FLAG_HOT_BACKWARD if hot else 0)
    W, m = fresh_params(cfg)
    W0, m0 = W.clone(), m.clone()
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device="cuda")
    meta = tbe.Meta(desc, N, weighted, with_pos=False)
    ws_f = tbe.workspace(desc, N, weighted, tbe.TBE_OP_FORWARD_PREPROCESS)
    ws_b = tbe.workspace(desc, N, weighted, tbe.TBE_OP_BACKWARD)

    def step():
        tbe.tbe_forward(desc, W, dev["indices"], dev["offsets"], dev["psw"], out, meta, ws_f)
        tbe.tbe_backward_adagrad(desc, W, m, dev["grad"], dev["indices"], dev["offsets"],
                                 dev["psw"], meta, cfg.lr, cfg.eps, ws_b)

    step()                                   # eager reference
    torch.cuda.synchronize()
    out_e, W_e, m_e = out.clone(), W.clone(), m.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        W.copy_(W0)
        m.copy_(m0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    for replay in range(3):
        W.copy_(W0)
        m.copy_(m0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(out_e)), f"replay {replay}: forward differs"
        assert torch.equal(_bits(W), _bits(W_e)), f"replay {replay}: weights differ"
        assert torch.equal(_bits(m), _bits(m_e)), f"replay {replay}: state differs"
