"""The one-launch MoE's hand-off between its gate/up and down workgroups.
Each down workgroup waits for its go word to receive one tagged release per
routed expert column (added by the gate/up workgroup that completes the
column) and keeps, next to it, the total it expected up to its last call.  A
release left over from an earlier call (one whose wait gave up) must not
start a later call's down pass early, and a go word holding a value no call
writes must be reported through the workspace's status word
(moe_workspace_status), not trusted.  The workspace words are set from the
host between ordinary calls; nothing waits for long."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu

# Workspace layout of moe_w4a16_gemv (see moe.hip): route header, one ticket
# word per 16 output rows (256-byte aligned), then the hand-off words: 128
# expert column counters (32 words apart), and per down workgroup (8 output
# rows) its go word and expected total, 16 words apart.
HEADER, SYNC_WORDS, GO_STRIDE, TAG = 16384, 32 * 128, 16, 0x9E3779B1
TOPK = 8


E, H, I = 64, 512, 512


def _u32(v):
    return np.uint32(v & 0xFFFFFFFF)


def _layout():
    sync = HEADER + (((H + 15) // 16 * 4 + 255) & ~255)
    go = [(sync + 4 * (SYNC_WORDS + GO_STRIDE * i)) // 4 for i in range((H + 7) // 8)]
    return go


def _experts():
    ex = synth.moe_quantized_experts(21, E, H, I)

    def glob(g):
        a = np.zeros((len(g), 4), np.float32)
        a[:, 0] = g
        return dev_f32(a)
    import nvfp4_w4a16_mtp_amd as nv
    dex = nv.NVFP4Experts(dev_u8(ex[0][0]), dev_u8(ex[0][1]), glob(ex[0][2]), dev_u8(ex[1][0]), dev_u8(ex[1][1]),
                          glob(ex[1][2]), dev_u8(ex[2][0]), dev_u8(ex[2][1]), glob(ex[2][2]))
    return ex, dex


def _words(ws):
    return ws.view(torch.int32)


def test_stale_release_does_not_start_a_later_call(orc):
    import nvfp4_w4a16_mtp_amd as nv
    ex, dex = _experts()
    x = synth.acts_bf16(22, 1, H)
    r = synth.router_logits(22, 1, E)
    ry, rids, _ = orc.moe(x, r, 8, *ex)
    ws = nv.moe_workspace(1, 8, dex, "cuda")
    go = torch.tensor(_layout(), dtype=torch.int64, device="cuda")
    for call in range(3):
        y, ids, _ = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), 8, dex, workspace=ws)
        assert nv.moe_workspace_status(ws) == 0
        assert np.array_equal(ids.cpu().numpy(), rids)
        assert_close(y.cpu().numpy(), ry, f"call {call}")
        w = _words(ws)
        # the one-launch path ran: every down workgroup received one tagged
        # release per expert column of every call, and expected as many
        done = _u32((call + 1) * TOPK * TAG)
        assert (w[go + 1].cpu().numpy().astype(np.uint32) == done).all()
        assert (w[go].cpu().numpy().astype(np.uint32) == done).all()
    # a call whose wait gave up (its expected total advanced) and whose
    # releases then landed late: the next call must wait for its own releases
    late = torch.tensor(np.array([_u32(4 * TOPK * TAG)]).view(np.int32)[0], device="cuda")
    w = _words(ws)
    w[go + 1] = late
    w[go] = late
    torch.cuda.synchronize()
    y, ids, _ = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), 8, dex, workspace=ws)
    assert nv.moe_workspace_status(ws) == 0
    assert_close(y.cpu().numpy(), ry, "after a late release")


def test_overwritten_go_word_is_reported(orc):
    import nvfp4_w4a16_mtp_amd as nv
    ex, dex = _experts()
    x = synth.acts_bf16(23, 1, H)
    r = synth.router_logits(23, 1, E)
    ry, _, _ = orc.moe(x, r, 8, *ex)
    ws = nv.moe_workspace(1, 8, dex, "cuda")
    go = _layout()
    _words(ws)[go[0]] = 1                       # a value no call writes (the old 0/1 flag)
    torch.cuda.synchronize()
    y, _, _ = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), 8, dex, workspace=ws)
    with pytest.raises(nv.NVFP4Error, match="overwritten"):
        nv.moe_workspace_status(ws)
    yh = y.cpu().numpy()
    assert np.isnan(yh[0, :8]).all()            # the rows of that down workgroup
    assert_close(yh[:, 8:], ry[:, 8:], "the other rows")
    assert nv.moe_workspace_status(ws) == 0     # read and cleared
    ws.zero_()                                  # the documented recovery
    y, _, _ = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), 8, dex, workspace=ws)
    assert nv.moe_workspace_status(ws) == 0
    assert_close(y.cpu().numpy(), ry, "after zero-filling")
