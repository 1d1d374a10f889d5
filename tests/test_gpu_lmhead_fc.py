"""GPU parity of lmhead_gemv_argmax_fc: the LM head's argmax, then the next
draft step's fc over [embedding row of the chosen token | hidden rest]
(deepseek_v4_mtp.rs `propose` feeds each draft into the next step's input;
mtp_head.rs `MtpHead` fields: `embed_from_argmax`, the fc).  At one row it
is one launch: the LM head's workgroups wait for the last one to publish
the id, then finish the fc.  Exact-arithmetic inputs (exact-family weights,
table and rest rows in {-3..3}) are compared with the oracle bit for bit;
random inputs give the two separate calls' out_idx and out_max bit for bit
and their fc output up to fp32 summation order.  Repeated calls on one
workspace and graph replays check that the published id is this call's."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _ints(seed, rows, cols):
    rng = np.random.default_rng([seed, 6])
    return synth.f32_to_bf16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32))


@pytest.mark.parametrize("fc_n,fc_k,hidden", [(2048, 4096, 2048), (512, 2048, 1024), (300, 4096, 4096)])
def test_exact_family_bit_exact(orc, fc_n, fc_k, hidden):
    import nvfp4_w4a16_mtp_amd as nv
    V, K = 5003, 2048
    h, codes, scales, g = synth.exact_family(720, 1, V, K)
    _, fcodes, fscales, fg = synth.exact_family(721, 1, fc_n, fc_k)
    table = _ints(722, V, hidden)
    rest = _ints(723, 1, fc_k - hidden)
    ridx, rmax = orc.lmhead_argmax(h, codes, scales, g)
    x = np.concatenate([orc.embed_rows(ridx, table), rest], axis=1)
    ry = orc.gemv(x, fcodes, fscales, fg)
    oi, om, y = nv.lmhead_gemv_argmax_fc(dev_bf16(h), _w(codes, scales, g), dev_bf16(table),
                                         dev_bf16(rest) if fc_k > hidden else None, _w(fcodes, fscales, fg))
    assert np.array_equal(oi.cpu().numpy(), ridx)
    assert np.array_equal(om.cpu().numpy().view(np.uint32), rmax.view(np.uint32))
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ry.view(np.uint32))


def _random_setup(V=32768, seed=730):
    import nvfp4_w4a16_mtp_amd as nv
    H = 2048
    w = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(seed, V, H)))
    fc = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(seed + 1, 2048, 2 * H)))
    table = dev_bf16(synth.acts_bf16(seed + 2, V, H))
    rest = dev_bf16(synth.acts_bf16(seed + 3, 8, H))
    return w, fc, table, rest


@pytest.mark.parametrize("bf16_keys", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_random_equals_the_two_calls(bf16_keys, out_dtype):
    import nvfp4_w4a16_mtp_amd as nv
    w, fc, table, rest = _random_setup()
    ws = nv.lmhead_workspace(1, w.n, "cuda")
    for call in range(4):
        h = dev_bf16(synth.acts_bf16(740 + call, 1, 2048))
        i0, m0 = nv.lmhead_gemv_argmax(h, w, bf16_keys=bf16_keys)
        y0 = nv.w4a16_gemv_embed(i0, table, rest[:1], fc, out_dtype=out_dtype)
        i1, m1, y1 = nv.lmhead_gemv_argmax_fc(h, w, table, rest[:1], fc, bf16_keys=bf16_keys, workspace=ws,
                                             out_dtype=out_dtype)
        assert torch.equal(i0, i1), f"call {call}"
        assert torch.equal(m0.view(torch.int32), m1.view(torch.int32))
        assert_close(y1.float().cpu().numpy(), y0.float().cpu().numpy(), f"call {call}")


def test_graph_replays_follow_each_draft():
    """Five chained calls in a graph, each on its own head input, replayed
    with eager work between: every replay's ids and fc rows are the eager
    ones (a published id from an earlier call would give a wrong fc row)."""
    import nvfp4_w4a16_mtp_amd as nv
    w, fc, table, rest = _random_setup(V=16384, seed=750)
    hs = [dev_bf16(synth.acts_bf16(760 + i, 1, 2048)) for i in range(5)]
    ws = nv.lmhead_workspace(1, w.n, "cuda")
    ids = torch.empty(5, dtype=torch.int32, device="cuda")
    mx = torch.empty(5, dtype=torch.float32, device="cuda")
    ys = torch.empty((5, 2048), dtype=torch.float32, device="cuda")

    def calls():
        for i in range(5):
            nv.lmhead_gemv_argmax_fc(hs[i], w, table, rest[:1], fc, workspace=ws, out_idx=ids[i:i + 1],
                                     out_max=mx[i:i + 1], out=ys[i:i + 1])
    torch.cuda.synchronize()   # the workspace is zero-filled before the stream's calls start
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        calls()
        torch.cuda.synchronize()
        ref = (ids.clone(), mx.clone(), ys.clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls()
    for rep in range(4):
        ids.fill_(-7)
        ys.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref[0]), f"replay {rep}"
        assert torch.equal(ys.view(torch.int32), ref[2].view(torch.int32)), f"replay {rep}"
    for i in range(5):   # and each against the separate calls
        i0, _ = nv.lmhead_gemv_argmax(hs[i], w)
        assert int(i0) == int(ref[0][i])
        y0 = nv.w4a16_gemv_embed(i0, table, rest[:1], fc)
        assert_close(ref[2][i:i + 1].cpu().numpy(), y0.cpu().numpy(), f"step {i}")


def test_two_rows_take_the_two_calls():
    import nvfp4_w4a16_mtp_amd as nv
    w, fc, table, rest = _random_setup(V=8192, seed=770)
    h = dev_bf16(synth.acts_bf16(771, 2, 2048))
    i0, m0 = nv.lmhead_gemv_argmax(h, w)
    y0 = nv.w4a16_gemv_embed(i0, table, rest[:2], fc)
    i1, m1, y1 = nv.lmhead_gemv_argmax_fc(h, w, table, rest[:2], fc)
    assert torch.equal(i0, i1) and torch.equal(m0.view(torch.int32), m1.view(torch.int32))
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))


@pytest.mark.parametrize("V,fc_n,fc_k", [
    (8192, 4000, 2048),    # more fc rows than the head's wavefronts take (7 x 256 CUs x 2): the two calls
    (300, 2048, 4096),     # a 19-workgroup head: too few wavefronts for the fc rows
    (8192, 1024, 3072),    # an fc width other than 2048 or 4096
    (8192, 2048, 2048)])   # fused, no rest part
def test_each_path_equals_the_two_calls(V, fc_n, fc_k):
    """Shapes on either side of the one-launch form's limits: the outputs are
    the two separate calls' (the id bit for bit, the fc row bit for bit when
    the call falls back to them, up to summation order when it fuses)."""
    import nvfp4_w4a16_mtp_amd as nv
    H = 2048
    w = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(780, V, H)))
    fc = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(781, fc_n, fc_k)))
    table = dev_bf16(synth.acts_bf16(782, V, H))
    rest = dev_bf16(synth.acts_bf16(783, 1, fc_k - H)) if fc_k > H else None
    h = dev_bf16(synth.acts_bf16(784, 1, H))
    i0, m0 = nv.lmhead_gemv_argmax(h, w)
    y0 = nv.w4a16_gemv_embed(i0, table, rest, fc)
    i1, m1, y1 = nv.lmhead_gemv_argmax_fc(h, w, table, rest, fc)
    assert torch.equal(i0, i1) and torch.equal(m0.view(torch.int32), m1.view(torch.int32))
    # one workgroup of 8 wavefronts per CU; wavefronts 1..7 take two fc rows each
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fused = fc_k in (2048, 4096) and fc_n <= 7 * min(cus, (V + 15) // 16) * 2
    if fused:
        assert_close(y1.cpu().numpy(), y0.cpu().numpy(), f"V={V} fc {fc_n}x{fc_k}")
    else:
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
