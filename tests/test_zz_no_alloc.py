"""lmhead_gemv_argmax_noalloc (C ABI): the LM-head argmax for callers that
cannot allocate, with its workspace in the library's static per-device
scratch.  Its results must equal lmhead_gemv_argmax's (a caller workspace,
the same kernels) bit for bit, on two calls in a row of which the second is
smaller, and the oracle's on the exact-arithmetic family.  Run alone in a
fresh process (the first call on the device sets the scratch up) and after
every other test."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _both(h, wd, v, bf16):
    import nvfp4_w4a16_mtp_amd as nv
    a_i, a_m = nv.lmhead_gemv_argmax_noalloc(dev_bf16(h), wd, vocab_rows=v, bf16_keys=bf16)
    b_i, b_m = nv.lmhead_gemv_argmax(dev_bf16(h), wd, vocab_rows=v, bf16_keys=bf16)
    a_i, a_m, b_i, b_m = (t.cpu().numpy() for t in (a_i, a_m, b_i, b_m))
    assert np.array_equal(a_i, b_i)
    assert np.array_equal(a_m.view(np.uint32), b_m.view(np.uint32))
    return a_i, a_m


@pytest.mark.parametrize("bf16", [False, True])
def test_two_calls_second_smaller_exact_family(orc, bf16):
    x, codes, scales, g = synth.exact_family(700, 8, 20000, 2048)
    wd = _w(codes, scales, g)
    for m, v in ((8, 0), (3, 5000)):             # second call: fewer rows, a shorter vocabulary
        idx, mx = _both(x[:m], wd, v, bf16)
        ridx, rmx = orc.lmhead_argmax(x[:m], codes, scales, g, vrows=v, flags=int(bf16))
        assert np.array_equal(idx, ridx) and np.array_equal(mx.view(np.uint32), rmx.view(np.uint32))


def test_config_head_planted_then_smaller(orc):
    """The 151936 x 2048 head at eight rows with planted winners, then one
    row over the first 32768 rows."""
    rng = np.random.default_rng(701)
    codes, scales, g = synth.quantized_domain_weight(rng, 151936, 2048)
    h = synth.acts_bf16(702, 8, 2048)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=703, n_near=4, dup=True, vrows=32768)
    wd = _w(codes, scales, g)
    idx, _ = _both(h, wd, 0, False)
    for i in range(8):
        assert idx[i] == min([info["star"][i]] + info["dups"][i])
    idx, _ = _both(h[:1], wd, 32768, False)
    assert idx[0] == min([info["star"][0]] + info["dups"][0])


def test_repeated_calls_and_a_graph(orc):
    """Back-to-back calls (the counters return to zero each time) and the
    call captured in a HIP graph, replayed with eager calls in between."""
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(704, 4, 9000, 1024)
    wd = _w(codes, scales, g)
    ridx, rmx = orc.lmhead_argmax(x, codes, scales, g)
    h = dev_bf16(x)
    oi = torch.empty(4, dtype=torch.int32, device="cuda")
    om = torch.empty(4, dtype=torch.float32, device="cuda")
    for _ in range(5):
        nv.lmhead_gemv_argmax_noalloc(h, wd, out_idx=oi, out_max=om)
    assert np.array_equal(oi.cpu().numpy(), ridx)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nv.lmhead_gemv_argmax_noalloc(h, wd, out_idx=oi, out_max=om)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            nv.lmhead_gemv_argmax_noalloc(h, wd, out_idx=oi, out_max=om)
    for _ in range(3):
        oi.fill_(-1)
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(oi.cpu().numpy(), ridx)
        assert np.array_equal(om.cpu().numpy().view(np.uint32), rmx.view(np.uint32))
        _both(x[:2], wd, 100, False)
