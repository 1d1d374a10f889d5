"""Repeated calls through the cross-workgroup hand-offs inside one launch: the
one-launch MoE (activations stored device-scope, column counters, per-column
releases into the down workgroups' go words), the LM head (per-workgroup
partials, the packed per-row maxima and the ticket of the last workgroup) and
the LM head with the next step's fc (the draft id published with the call's
count to every workgroup).  All three rely on the ordering of device-scope relaxed atomics and coherent
loads and stores on gfx950 rather than on release/acquire fences, so this
replays thousands of calls from HIP graphs -- the bench's Qwen shapes,
inputs rotating between calls -- and requires every one of them to be bit
for bit the eager call on the same inputs (eager work and a synchronization
between replays)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

CALLS = 64      # calls per graph
REPLAYS = 150   # replays: 9600 calls
ROT = 16        # distinct inputs, rotated over the calls


def _randn(gen, shape, std=1.0, dtype=torch.bfloat16):
    t = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
    return (t * std).to(dtype)


def _bits(t):
    return t.view(torch.int32)


def _soak(graph, outs, refs):
    """Replays `graph`; counts outputs whose bits differ from refs."""
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(REPLAYS):
        graph.replay()
        for o, r in zip(outs, refs):
            bad += (_bits(o) != _bits(r)).reshape(o.shape[0], -1).any(dim=1).sum()
        torch.cuda.synchronize()
    return int(bad.item())


def test_moe_one_launch_replays_match_eager():
    import nvfp4_w4a16_mtp_amd as nv
    E, H, I, K = 256, 2048, 1024, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(900)
    parts = []
    for rows, cols in ((I, H), (I, H), (H, I)):
        q = nv.nvfp4_quantize(_randn(gen, (E * rows, cols), 0.02))
        parts += [q.codes.view(E, rows, cols // 2), q.scales.view(E, rows, cols // 16),
                  q.glob.repeat(E, 1).contiguous()]
    ex = nv.NVFP4Experts(*parts)
    x = _randn(gen, (1, H))
    routers = _randn(gen, (ROT, E), dtype=torch.float32)
    ws = nv.moe_workspace(1, K, ex, "cuda")
    ref_y, ref_ids = [], []
    for r in range(ROT):
        y, ids, _ = nv.moe_w4a16_gemv(x, routers[r:r + 1], K, ex, workspace=ws)
        ref_y.append(y.clone())
        ref_ids.append(ids.clone())
    assert nv.moe_workspace_status(ws) == 0
    ys = torch.empty((CALLS, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((CALLS, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((CALLS, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()   # the reference calls have finished before the stream's calls start
    s = torch.cuda.Stream()

    def calls():
        for i in range(CALLS):
            r = i % ROT
            nv.moe_w4a16_gemv(x, routers[r:r + 1], K, ex, workspace=ws, out=ys[i:i + 1], topk_ids=ids[i:i + 1],
                              topk_w=wts[i:i + 1])
    with torch.cuda.stream(s):
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    want_y = torch.cat([ref_y[i % ROT] for i in range(CALLS)])
    want_ids = torch.cat([ref_ids[i % ROT] for i in range(CALLS)])
    assert _soak(g, [ys, ids], [want_y, want_ids]) == 0
    assert nv.moe_workspace_status(ws) == 0


def test_lmhead_replays_match_eager():
    import nvfp4_w4a16_mtp_amd as nv
    V, H = 151936, 2048
    gen = torch.Generator(device="cuda")
    gen.manual_seed(901)
    w = nv.nvfp4_quantize(_randn(gen, (V, H), 0.02))
    hs = _randn(gen, (ROT, H))
    ws = nv.lmhead_workspace(1, V, "cuda")
    ref_i, ref_m = [], []
    for r in range(ROT):
        i, m = nv.lmhead_gemv_argmax(hs[r:r + 1], w, workspace=ws)
        ref_i.append(i.clone())
        ref_m.append(m.clone())
    oi = torch.empty(CALLS, dtype=torch.int32, device="cuda")
    om = torch.empty(CALLS, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()   # the reference calls have finished before the stream's calls start
    s = torch.cuda.Stream()

    def calls():
        for i in range(CALLS):
            r = i % ROT
            nv.lmhead_gemv_argmax(hs[r:r + 1], w, workspace=ws, out_idx=oi[i:i + 1], out_max=om[i:i + 1])
    with torch.cuda.stream(s):
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    want_i = torch.cat([ref_i[i % ROT] for i in range(CALLS)]).reshape(CALLS, 1)
    want_m = torch.cat([ref_m[i % ROT] for i in range(CALLS)]).reshape(CALLS, 1)
    assert _soak(g, [oi.reshape(CALLS, 1), om.reshape(CALLS, 1)], [want_i, want_m]) == 0


def test_lmhead_fc_replays_match_eager():
    """The LM head with the next step's fc in one launch: the last workgroup
    publishes the draft id with the call's count, the others wait for the
    count to change and finish the fc over that id's embedding row."""
    import nvfp4_w4a16_mtp_amd as nv
    V, H = 151936, 2048
    gen = torch.Generator(device="cuda")
    gen.manual_seed(902)
    w = nv.nvfp4_quantize(_randn(gen, (V, H), 0.02))
    fc = nv.nvfp4_quantize(_randn(gen, (H, 2 * H), 0.02))
    table = _randn(gen, (V, H))
    hs = _randn(gen, (ROT, H))
    rest = _randn(gen, (ROT, H))
    ws = nv.lmhead_workspace(1, V, "cuda")
    ref_i, ref_y = [], []
    for r in range(ROT):
        i, _, y = nv.lmhead_gemv_argmax_fc(hs[r:r + 1], w, table, rest[r:r + 1], fc, workspace=ws)
        ref_i.append(i.clone())
        ref_y.append(y.clone())
    oi = torch.empty(CALLS, dtype=torch.int32, device="cuda")
    om = torch.empty(CALLS, dtype=torch.float32, device="cuda")
    ys = torch.empty((CALLS, H), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()   # the reference calls have finished before the stream's calls start
    s = torch.cuda.Stream()

    def calls():
        for i in range(CALLS):
            r = i % ROT
            nv.lmhead_gemv_argmax_fc(hs[r:r + 1], w, table, rest[r:r + 1], fc, workspace=ws, out_idx=oi[i:i + 1],
                                     out_max=om[i:i + 1], out=ys[i:i + 1])
    with torch.cuda.stream(s):
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    want_i = torch.cat([ref_i[i % ROT] for i in range(CALLS)]).reshape(CALLS, 1)
    want_y = torch.cat([ref_y[i % ROT] for i in range(CALLS)])
    assert _soak(g, [oi.reshape(CALLS, 1), ys], [want_i, want_y]) == 0
