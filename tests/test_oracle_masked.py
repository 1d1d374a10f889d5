"""Pins for the oracle's grammar-masked LM-head argmax and the embedding
gather (CPU).

The masked scan is the one of deepseek_v4_mtp.rs (`argmax_grammar_masked`):
token r is allowed when bit r % 32 of mask word r / 32 is set (words past the
mask allow nothing), the ascending strict-greater scan runs over the allowed
tokens from index 0 and -inf, and an empty allowed set returns 0.  Pins: a
brute-force Python scan over logits computed independently in numpy, the
unmasked case against the already pinned argmax and log-probability, the
empty and single-token sets, a short mask, and an independent log-sum-exp
(scipy) over the allowed keys.
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


def _mask_bits(allowed):
    """bool [m][v] -> uint32 [m][ceil(v / 32)]"""
    m, v = allowed.shape
    words = np.zeros((m, (v + 31) // 32), np.uint32)
    for i in range(m):
        for r in np.flatnonzero(allowed[i]):
            words[i, r // 32] |= np.uint32(1) << np.uint32(r % 32)
    return words


def _scan(keys, allowed):
    best, bi = -np.inf, 0
    for r in range(len(keys)):
        if allowed[r] and keys[r] > best:
            best, bi = keys[r], r
    return bi


def _head(seed, m, v, k=128):
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(seed), v, k)
    return synth.acts_bf16(seed + 1, m, k), codes, scales, np.float32(g * 300)


@pytest.mark.parametrize("seed,m,v,density,flags", [(0, 1, 300, 0.5, 0), (1, 4, 1000, 0.05, 0), (2, 3, 77, 0.9, 1),
                                                     (3, 8, 513, 0.01, 1)])
def test_brute_force_scan(orc, seed, m, v, density, flags):
    h, codes, scales, g = _head(seed, m, v)
    rng = np.random.default_rng(seed + 100)
    allowed = rng.random((m, v)) < density
    if m > 1:
        allowed[0, :] = False                                   # a row with nothing allowed
    keys = _logits_numpy(h, codes, scales, g).astype(np.float64)
    logits = keys.copy()
    if flags:
        keys = torch.from_numpy(keys.astype(np.float32)).to(torch.bfloat16).double().numpy()
    idx, mx, lp = orc.lmhead_masked(h, codes, scales, g, mask=_mask_bits(allowed), flags=flags)
    for i in range(m):
        want = _scan(keys[i], allowed[i])
        assert idx[i] == want
        assert abs(mx[i] - logits[i, want]) <= 1e-6 * max(1.0, abs(logits[i, want]))
        if allowed[i].any():
            ref = keys[i, want] - logsumexp(keys[i][allowed[i]])
            assert abs(lp[i] - ref) < 1e-6
        else:
            assert idx[i] == 0 and np.isnan(lp[i])


def test_unmasked_equals_argmax_and_logprob(orc):
    h, codes, scales, g = _head(10, 5, 700)
    idx, mx, lp = orc.lmhead_masked(h, codes, scales, g)
    ridx, rmx = orc.lmhead_argmax(h, codes, scales, g)
    assert np.array_equal(idx, ridx) and np.array_equal(mx.view(np.uint32), rmx.view(np.uint32))
    assert np.allclose(lp, orc.lmhead_logprob(h, codes, scales, g), rtol=0, atol=1e-12)
    allowed = np.ones((5, 700), bool)
    idx2, mx2, lp2 = orc.lmhead_masked(h, codes, scales, g, mask=_mask_bits(allowed))
    assert np.array_equal(idx2, idx) and np.array_equal(lp2, lp)


def test_single_allowed_token(orc):
    h, codes, scales, g = _head(20, 2, 400)
    allowed = np.zeros((2, 400), bool)
    allowed[0, 321] = True
    allowed[1, 0] = True
    idx, _, lp = orc.lmhead_masked(h, codes, scales, g, mask=_mask_bits(allowed))
    assert list(idx) == [321, 0] and np.all(lp == 0.0)


def test_short_mask_allows_nothing_beyond(orc):
    h, codes, scales, g = _head(30, 1, 200)
    keys = _logits_numpy(h, codes, scales, g)[0]
    allowed = np.ones((1, 64), bool)                            # two words: rows 0..63
    idx, _, lp = orc.lmhead_masked(h, codes, scales, g, mask=_mask_bits(allowed))
    assert idx[0] == int(np.argmax(keys[:64]))
    assert abs(lp[0] - (keys[idx[0]] - logsumexp(keys[:64].astype(np.float64)))) < 1e-6


def test_embed_rows(orc):
    rng = np.random.default_rng(40)
    table = rng.integers(0, 65536, size=(1000, 48), dtype=np.uint16)
    idx = np.array([0, 999, 5, -1, 1000, 5], np.int32)
    out = orc.embed_rows(idx, table)
    assert np.array_equal(out[[0, 1, 2, 5]], table[[0, 999, 5, 5]])
    assert not out[3].any() and not out[4].any()
