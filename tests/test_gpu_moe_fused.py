"""GPU parity of the one-launch MoE (gate/up and the row-owner down pass in
one grid, handing off through column counters and tagged go words in the
workspace): a
run of calls on one workspace with a different routing each time, and a
captured graph replayed several times with eager work in between, every
result against the oracle.  A wrong reset of the hand-off words would let a
later call's down pass read activations before they exist."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_f32
from tests.test_gpu_moe import _dev_experts

pytestmark = pytest.mark.gpu

H, I, E, TOPK = 2048, 512, 64, 8   # m = 1: one launch holding every workgroup; m = 2: two launches, the ticket down pass


@pytest.fixture(scope="module")
def experts():
    ex = synth.moe_quantized_experts(60, E, H, I)
    return ex, _dev_experts(*ex)


@pytest.mark.parametrize("m", [1, 2])
def test_consecutive_calls_one_workspace(orc, experts, m):
    import nvfp4_w4a16_mtp_amd as nv
    ex, dex = experts
    ws = nv.moe_workspace(m, TOPK, dex, "cuda")
    for call in range(6):
        x = synth.acts_bf16(61 + 10 * m + call, m, H)
        r = synth.router_logits(62 + 10 * m + call, m, E)
        y, ids, w = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), TOPK, dex, workspace=ws)
        ry, rids, rw = orc.moe(x, r, TOPK, *ex)
        assert np.array_equal(ids.cpu().numpy(), rids), f"call {call}"
        assert_close(w.cpu().numpy(), rw, f"weights, call {call}")
        assert_close(y.cpu().numpy(), ry, f"output, call {call}")


def test_graph_replays(orc, experts):
    import nvfp4_w4a16_mtp_amd as nv
    ex, dex = experts
    m = 1
    ws = nv.moe_workspace(m, TOPK, dex, "cuda")
    xs = [synth.acts_bf16(70 + i, m, H) for i in range(2)]
    rs = [synth.router_logits(72 + i, m, E) for i in range(2)]
    refs = [orc.moe(xs[i], rs[i], TOPK, *ex) for i in range(2)]
    xin, rin = dev_bf16(xs[0]), dev_f32(rs[0])
    y = torch.empty((m, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((m, TOPK), dtype=torch.int32, device="cuda")
    w = torch.empty((m, TOPK), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()   # the workspace is zero-filled before the stream's calls start
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nv.moe_w4a16_gemv(xin, rin, TOPK, dex, workspace=ws, out=y, topk_ids=ids, topk_w=w)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(3):
                nv.moe_w4a16_gemv(xin, rin, TOPK, dex, workspace=ws, out=y, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 2
        xin.copy_(dev_bf16(xs[i]))
        rin.copy_(dev_f32(rs[i]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ry, rids, rw = refs[i]
        assert np.array_equal(ids.cpu().numpy(), rids), f"replay {rep}"
        assert_close(y.cpu().numpy(), ry, f"output, replay {rep}")
        # eager work between replays
        y2, _, _ = nv.moe_w4a16_gemv(dev_bf16(xs[1 - i]), dev_f32(rs[1 - i]), TOPK, dex, workspace=ws)
        assert_close(y2.cpu().numpy(), refs[1 - i][0], f"eager output after replay {rep}")
