"""The one-token MoE with phase timestamps (moe_w4a16_gemv_trace): the same
kernel as moe_w4a16_gemv, so its outputs must be that call's bit for bit
(and the oracle's), every event of every workgroup must be recorded in
order, and the timestamps must show the hand-off's ordering: no down
workgroup sees its go word before every gate/up workgroup has stored its
activations (a release precedes nothing it covers).  The clock is the GPU's
100 MHz constant counter, shared by every compute unit."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_f32
from tests.test_gpu_moe import _dev_experts

pytestmark = pytest.mark.gpu

H, I, E, TOPK = 2048, 512, 64, 8


@pytest.fixture(scope="module")
def experts():
    ex = synth.moe_quantized_experts(80, E, H, I)
    return ex, _dev_experts(*ex)


def test_trace_matches_the_plain_call_and_orders_the_hand_off(orc, experts):
    import nvfp4_w4a16_mtp_amd as nv
    ex, dex = experts
    ev, groups = nv.moe_trace_events(TOPK, dex)
    gate_up = (I + 15) // 16 * TOPK
    assert (ev, groups) == (6, gate_up + (H + 7) // 8)
    ws = nv.moe_workspace(1, TOPK, dex, "cuda")
    for call in range(3):
        x = synth.acts_bf16(81 + call, 1, H)
        r = synth.router_logits(82 + call, 1, E)
        y0, ids0, w0 = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), TOPK, dex, workspace=ws)
        trace = torch.full((ev, groups), -1, dtype=torch.int64, device="cuda")
        y1, ids1, w1 = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), TOPK, dex, workspace=ws, trace=trace)
        assert nv.moe_workspace_status(ws) == 0
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), f"call {call}"
        assert torch.equal(ids0, ids1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
        ry, rids, _ = orc.moe(x, r, TOPK, *ex)
        assert np.array_equal(ids1.cpu().numpy(), rids)
        assert_close(y1.cpu().numpy(), ry, f"call {call}")
        t = trace.cpu().numpy()
        gu, dn = t[:4, :gate_up], t[:, gate_up:]
        assert (t[4:, :gate_up] == -1).all()              # gate/up workgroups record events 0..3 only
        assert (gu > 0).all() and (dn > 0).all()
        assert (np.diff(gu, axis=0) >= 0).all() and (np.diff(dn, axis=0) >= 0).all()
        # every go word is seen after the last activation store of the call
        assert dn[2].min() >= gu[2].max(), (dn[2].min(), gu[2].max())
        # and the whole launch spans microseconds, not seconds (no wait ran out)
        assert (dn[5].max() - gu[0].min()) < 100 * 1000   # 1 ms at 100 MHz


def test_trace_needs_the_one_launch_form(experts):
    import nvfp4_w4a16_mtp_amd as nv
    _, dex = experts
    x = dev_bf16(synth.acts_bf16(90, 2, H))
    r = dev_f32(synth.router_logits(91, 2, E))
    ev, groups = nv.moe_trace_events(TOPK, dex)
    trace = torch.zeros((ev, groups), dtype=torch.int64, device="cuda")
    with pytest.raises(nv.NVFP4Error, match="one token"):
        nv.moe_w4a16_gemv(x, r, TOPK, dex, trace=trace)
