"""GPU parity: lmhead_gemv_argmax_logprob (C ABI) vs the oracle's top-1
log-probability.  The index and max logit equal those of lmhead_gemv_argmax
bit for bit (same scoring, same combine); the log-probability is within
|d| <= 1e-3 + 2e-3 |ref| of the oracle's fp64 value, on random heads, the
full 151936 x 2048 head with planted rows, the bf16-key mode, a reduced
vocabulary and the equal-logit closed form."""
import ctypes
import math

import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _both(h, wd, vrows=0, bf16=False):
    import nvfp4_w4a16_mtp_amd as nv
    hd = dev_bf16(h)
    i0, m0 = nv.lmhead_gemv_argmax(hd, wd, vocab_rows=vrows, bf16_keys=bf16)
    i1, m1, lp = nv.lmhead_gemv_argmax_logprob(hd, wd, vocab_rows=vrows, bf16_keys=bf16)
    i0, m0, i1, m1 = (t.cpu().numpy() for t in (i0, m0, i1, m1))
    assert np.array_equal(i0, i1)
    assert np.array_equal(m0.view(np.uint32), m1.view(np.uint32))
    return i1, m1, lp.cpu().numpy()


@pytest.mark.parametrize("m,v,k,bf16", [(1, 3000, 512, False), (3, 4097, 2048, False), (8, 2500, 2048, True),
                                         (5, 700, 1024, True)])
def test_random_heads(orc, m, v, k, bf16):
    rng = np.random.default_rng([m, v, k])
    codes, scales, g = synth.quantized_domain_weight(rng, v, k)
    g = np.float32(g * 400.0)                             # logits spread over several units
    h = synth.acts_bf16(7 + m, m, k)
    _, _, lp = _both(h, _w(codes, scales, g), bf16=bf16)
    ref = orc.lmhead_logprob(h, codes, scales, g, flags=int(bf16))
    assert_close(lp, ref, f"logprob m={m} v={v}")
    assert (lp <= 1e-6).all() and (lp >= -math.log(v) - 1e-3).all()


def test_reduced_vocabulary(orc):
    v, k = 5000, 2048
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(41), v, k)
    g = np.float32(g * 400.0)
    h = synth.acts_bf16(42, 4, k)
    _, _, lp = _both(h, _w(codes, scales, g), vrows=1234)
    assert_close(lp, orc.lmhead_logprob(h, codes, scales, g, vrows=1234), "reduced V")


def test_equal_logits_closed_form():
    import nvfp4_w4a16_mtp_amd as nv
    v, k = 32768, 2048
    wd = nv.NVFP4Weight.from_parts(torch.zeros((v, k // 2), dtype=torch.uint8, device="cuda"),
                                   torch.full((v, k // 16), 0x38, dtype=torch.uint8, device="cuda"), 1.0)
    h = synth.acts_bf16(3, 8, k)
    idx, mx, lp = _both(h, wd)
    assert (idx == 0).all() and (mx == 0).all()
    assert np.allclose(lp, -math.log(v), rtol=2e-6, atol=0)


@pytest.mark.parametrize("m", [1, 8])
def test_full_head_planted(orc, m):
    """The 151936 x 2048 head of the workload with planted winners."""
    import nvfp4_w4a16_mtp_amd as nv
    v, k = 151936, 2048
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(77), v, k)
    g = np.float32(g * 400.0)
    h = synth.acts_bf16(78, m, k)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=79, n_near=4)
    idx, _, lp = _both(h, _w(codes, scales, g))
    assert list(idx) == [info["star"][i] for i in range(m)]
    assert_close(lp, orc.lmhead_logprob(h, codes, scales, g), f"full head m={m}")


def test_null_logprob_is_an_error():
    import nvfp4_w4a16_mtp_amd as nv
    wd = nv.NVFP4Weight.from_parts(torch.zeros((64, 16), dtype=torch.uint8, device="cuda"),
                                   torch.zeros((64, 2), dtype=torch.uint8, device="cuda"), 1.0)
    h = torch.zeros((1, 32), dtype=torch.bfloat16, device="cuda")
    ws = nv.lmhead_workspace(1, 64, "cuda")
    oi = torch.empty(1, dtype=torch.int32, device="cuda")
    om = torch.empty(1, dtype=torch.float32, device="cuda")
    d = wd.desc()
    rc = nv.lib().lmhead_gemv_argmax_logprob(ctypes.c_void_p(h.data_ptr()), 1, ctypes.byref(d), 0,
                                             ctypes.c_void_p(oi.data_ptr()), ctypes.c_void_p(om.data_ptr()), None,
                                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), 0, None)
    assert rc != 0 and b"out_logprob" in nv.lib().nvfp4_mtp_last_error()
