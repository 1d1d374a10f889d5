"""Repeated calls on one workspace (the ticket counters must return to zero)
and HIP-graph capture of a draft step: every replay, with eager work and
synchronizations in between, must equal the eager result bit for bit."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


def _experts(seed, E, H, I):
    import nvfp4_w4a16_mtp_amd as nv
    ex = synth.moe_quantized_experts(seed, E, H, I)

    def glob(g):
        a = np.zeros((len(g), 4), np.float32)
        a[:, 0] = g
        return dev_f32(a)
    return nv.NVFP4Experts(dev_u8(ex[0][0]), dev_u8(ex[0][1]), glob(ex[0][2]), dev_u8(ex[1][0]), dev_u8(ex[1][1]),
                           glob(ex[1][2]), dev_u8(ex[2][0]), dev_u8(ex[2][1]), glob(ex[2][2]))


def test_workspace_reuse(orc):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(1, 4, 9000, 512)
    wd = nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g))
    ws = nv.lmhead_workspace(4, 9000, "cuda")
    ref_idx, ref_max = orc.lmhead_argmax(x, codes, scales, g)
    for vrows in (9000, 100, 9000, 5000, 9000):
        idx, mx = nv.lmhead_gemv_argmax(dev_bf16(x), wd, vocab_rows=vrows, workspace=ws)
        r_idx, r_max = orc.lmhead_argmax(x, codes, scales, g, vrows=vrows)
        assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert int(ws[:4].view(torch.int32).item()) == 0


def test_graph_replays_match_eager():
    import nvfp4_w4a16_mtp_amd as nv
    dev = torch.device("cuda")
    M = 4
    wq = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(1, 1024, 2048)))
    wl = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(2, 20000, 2048)))
    ex = _experts(3, 64, 2048, 1024)
    x = dev_bf16(synth.acts_bf16(4, M, 2048))
    r = dev_f32(synth.router_logits(4, M, 64))
    y = torch.empty((M, 1024), dtype=torch.float32, device=dev)
    ym = torch.empty((M, 2048), dtype=torch.float32, device=dev)
    ids = torch.empty((M, 8), dtype=torch.int32, device=dev)
    wts = torch.empty((M, 8), dtype=torch.float32, device=dev)
    oi = torch.empty(M, dtype=torch.int32, device=dev)
    om = torch.empty(M, dtype=torch.float32, device=dev)
    mws = nv.moe_workspace(M, 8, ex, dev)
    lws = nv.lmhead_workspace(M, 20000, dev)

    def step():
        nv.w4a16_gemv(x, wq, out=y)
        nv.moe_w4a16_gemv(x, r, 8, ex, workspace=mws, out=ym, topk_ids=ids, topk_w=wts)
        nv.lmhead_gemv_argmax(x, wl, workspace=lws, out_idx=oi, out_max=om)

    torch.cuda.synchronize()   # the workspaces are zero-filled before the stream's calls start
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, ym, ids, wts, oi, om)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(5):
        for t in (y, ym, ids, wts, oi, om):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((y, ym, ids, wts, oi, om), eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        with torch.cuda.stream(s):
            step()                       # eager work between replays
        torch.cuda.synchronize()
