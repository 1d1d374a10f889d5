"""Pins for the oracle's top-1 log-probability of the LM-head argmax (CPU).

lp = key[argmax] - log(sum_r exp(key[r])) over the scored rows, with the keys
the argmax compares (fp32 logits, or their bf16 rounding).  Pins: closed
forms (equal logits give -log V; one planted logit L among zeros gives
L - log(e^L + V - 1); a one-row vocabulary gives 0), an independent
log-sum-exp (scipy) over logits computed independently in numpy, the
bf16-key variant, and the non-finite cases.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from tests import synth

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _logits_numpy(h, codes, scales, g_dec):
    k = h.shape[1]
    c = np.empty((codes.shape[0], k), np.int64)
    c[:, 0::2], c[:, 1::2] = codes & 15, codes >> 4
    W = E2M1[c & 7] * np.where(c & 8, -1.0, 1.0) * np.repeat(E4M3[scales], 16, axis=1)
    return (synth.bf16_bits_to_f32(h).astype(np.float64) @ W.T * float(g_dec)).astype(np.float32)


@pytest.mark.parametrize("v,vrows", [(4096, 0), (4096, 1000), (37, 0)])
def test_equal_logits_give_minus_log_v(orc, v, vrows):
    k = 64
    h = synth.acts_bf16(1, 3, k)
    codes = np.zeros((v, k // 2), np.uint8)
    scales = np.full((v, k // 16), 0x38, np.uint8)
    lp = orc.lmhead_logprob(h, codes, scales, 1.0, vrows=vrows)
    vv = v if vrows == 0 else vrows
    assert np.allclose(lp, -math.log(vv), rtol=0, atol=1e-12)


def test_planted_logit_closed_form(orc):
    k, v = 64, 500
    h = synth.f32_to_bf16_bits(np.ones((1, k), np.float32))
    codes = np.zeros((v, k // 2), np.uint8)
    scales = np.full((v, k // 16), 0x38, np.uint8)       # 1.0
    codes[123, :] = 0x22                                  # +1.0 everywhere: logit = k * g
    g = 2.0 ** -4
    L = k * g
    lp = orc.lmhead_logprob(h, codes, scales, g)
    assert abs(lp[0] - (L - math.log(math.exp(L) + v - 1))) < 1e-12
    # the same row planted negative: the argmax is a zero row
    codes[123, :] = 0xAA
    lp = orc.lmhead_logprob(h, codes, scales, g)
    assert abs(lp[0] - (0.0 - math.log(math.exp(-L) + v - 1))) < 1e-12


def test_single_row_vocabulary_is_zero(orc):
    k = 32
    h = synth.acts_bf16(2, 2, k)
    codes = synth.quantized_domain_weight(np.random.default_rng(5), 8, k)[0]
    scales = np.full((8, k // 16), 0x40, np.uint8)
    lp = orc.lmhead_logprob(h, codes, scales, 1e-2, vrows=1)
    assert np.all(lp == 0.0)


@pytest.mark.parametrize("seed,m,v,flags", [(0, 1, 700, 0), (1, 4, 2049, 0), (2, 3, 513, 1), (3, 8, 64, 1)])
def test_independent_logsumexp(orc, seed, m, v, flags):
    k = 256
    rng = np.random.default_rng(seed)
    codes, scales, g = synth.quantized_domain_weight(rng, v, k)
    g = np.float32(g * 300.0)                             # logits of order 1
    h = synth.acts_bf16(seed + 10, m, k)
    keys = _logits_numpy(h, codes, scales, g).astype(np.float64)
    if flags:
        keys = torch.from_numpy(keys.astype(np.float32)).to(torch.bfloat16).double().numpy()
    lp = orc.lmhead_logprob(h, codes, scales, g, flags=flags)
    idx, _ = orc.lmhead_argmax(h, codes, scales, g, flags=flags)
    for i in range(m):
        want = keys[i, idx[i]] - logsumexp(keys[i])
        # the oracle's keys are the fp32 rounding of the exact dot product;
        # numpy's fp64 matmul can differ by an fp32 ulp in the rare case of a
        # double rounding -- far below this bound
        assert abs(lp[i] - want) < 1e-6, (i, lp[i], want)
        assert lp[i] <= 1e-12


def test_argmax_has_the_largest_logprob(orc):
    """lp of the selected row is max over rows of key[r] - lse, i.e. lp >= -log V."""
    k, v = 128, 333
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(9), v, k)
    h = synth.acts_bf16(19, 5, k)
    lp = orc.lmhead_logprob(h, codes, scales, np.float32(g * 500))
    assert np.all(lp <= 0.0) and np.all(lp >= -math.log(v))


def test_nonfinite(orc):
    k = 32
    scales = np.full((4, k // 16), 0x38, np.uint8)
    codes = np.full((4, k // 2), 0x11, np.uint8)
    h = synth.f32_to_bf16_bits(np.ones((1, k), np.float32))
    assert np.isnan(orc.lmhead_logprob(h, codes, scales, np.float32(np.nan))[0])
    hi = synth.f32_to_bf16_bits(np.array([[np.inf] + [0.0] * (k - 1)], np.float32))
    codes = np.zeros((4, k // 2), np.uint8)
    codes[1, 0] = 0x02                                     # +inf logit
    assert np.isnan(orc.lmhead_logprob(hi, codes, scales, np.float32(1.0))[0])
