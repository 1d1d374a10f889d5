"""Pins for the oracle's LM-head GEMV + argmax (CPU only).

The selection rule is the CPU scan of deepseek_v4_mtp.rs
(`argmax_grammar_masked`): ascending, strict greater-than, start at -inf and
index 0, so the lowest index wins among equal maxima.  The reduced-vocab head
scores rows [0, V) (new.rs `MtpHead::new`, effective vocab; deepseek_v4_mtp.rs
`forward_one`).  Pins: a brute-force scan over logits computed independently,
closed-form planted rows, exact duplicates, bf16-key mode, NaN / -inf rows.
"""
import numpy as np
import pytest
import torch

from tests import synth
plant_rows = synth.plant_lmhead_rows

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _scan(keys):
    best, bi = -np.inf, 0
    for i, v in enumerate(keys):
        if v > best:
            best, bi = v, i
    return bi


def _logits_numpy(h, codes, scales, g_dec):
    n = codes.shape[0]
    k = h.shape[1]
    c = np.empty((n, k), np.int64)
    c[:, 0::2], c[:, 1::2] = codes & 15, codes >> 4
    W = E2M1[c & 7] * np.where(c & 8, -1.0, 1.0) * np.repeat(E4M3[scales], 16, axis=1)
    return (synth.bf16_bits_to_f32(h).astype(np.float64) @ W.T * float(g_dec)).astype(np.float32)


@pytest.mark.parametrize("seed,m,v", [(0, 1, 300), (1, 4, 513), (2, 8, 64)])
def test_scan_semantics_random(orc, seed, m, v):
    w = synth.weight_bf16(seed, v, 256)
    h = synth.acts_bf16(seed, m, 256)
    codes, scales, glob = orc.quantize(w)
    idx, mx, logits, _ = orc.lmhead_argmax(h, codes, scales, glob[0], want_logits=True)
    ref = _logits_numpy(h, codes, scales, glob[0])
    assert np.abs(logits - ref).max() <= 1e-6 * np.abs(ref).max()
    for i in range(m):
        assert idx[i] == _scan(logits[i]) and mx[i] == logits[i, idx[i]]


def test_reduced_vocab_is_prefix(orc):
    w = synth.weight_bf16(3, 700, 128)
    h = synth.acts_bf16(3, 4, 128)
    codes, scales, glob = orc.quantize(w)
    _, _, full, _ = orc.lmhead_argmax(h, codes, scales, glob[0], want_logits=True)
    for v in (1, 37, 500, 700, 5000):
        idx, mx = orc.lmhead_argmax(h, codes, scales, glob[0], vrows=v)
        vv = min(v, 700)
        for i in range(4):
            assert idx[i] == _scan(full[i, :vv])


def test_planted_closed_form_and_ties(orc):
    """A planted row (codes 7*sign(x), scale byte S everywhere) scores
    6 * e4m3(S) * g_dec * sum|x| exactly enough to beat every random row;
    exact duplicates resolve to the lowest index; near-tie copies lose by a
    closed-form margin."""
    v, k, m = 2000, 256, 3
    w = synth.weight_bf16(4, v, k)
    h = synth.acts_bf16(4, m, k)
    codes, scales, glob = orc.quantize(w)
    info = plant_rows(codes, scales, h, seed=4, n_near=4, dup=True)
    idx, mx, logits, _ = orc.lmhead_argmax(h, codes, scales, glob[0], want_logits=True)
    hf = synth.bf16_bits_to_f32(h).astype(np.float64)
    for i in range(m):
        star, dups = info["star"][i], info["dups"][i]
        sf = E4M3[info["scale_byte"]]
        closed = 6.0 * sf * float(glob[0]) * np.abs(hf[i]).sum()
        assert abs(logits[i, star] - closed) <= 1e-6 * closed
        assert idx[i] == min([star] + list(dups))
        for r, kk in zip(info["near"][i], info["near_k"][i]):
            margin = 2.0 * sf * float(glob[0]) * abs(hf[i, kk])
            assert abs((logits[i, star] - logits[i, r]) - margin) <= 1e-5 * closed


def test_bf16_key_mode(orc):
    """flags bit0 compares bf16-rounded logits: among rows whose logits round
    to the same bf16 value the lowest index wins."""
    w = synth.weight_bf16(5, 800, 128)
    h = synth.acts_bf16(5, 2, 128)
    codes, scales, glob = orc.quantize(w)
    _, _, logits, _ = orc.lmhead_argmax(h, codes, scales, glob[0], want_logits=True)
    idx, mx = orc.lmhead_argmax(h, codes, scales, glob[0], flags=1)
    keys = torch.from_numpy(logits).to(torch.bfloat16).float().numpy()
    for i in range(2):
        assert idx[i] == _scan(keys[i]) and mx[i] == logits[i, idx[i]]


def test_nonfinite_rows(orc):
    """NaN logits never win; an all-NaN head returns index 0; +inf wins at its
    first occurrence; -0 and +0 compare equal (first one kept)."""
    k = 32
    h = synth.f32_to_bf16_bits(np.ones((1, k), np.float32))
    scales = np.full((4, k // 16), 0x38, np.uint8)
    # g_dec = NaN makes every logit NaN
    codes = np.full((4, k // 2), 0x11, np.uint8)
    idx, mx = orc.lmhead_argmax(h, codes, scales, np.float32(np.nan))
    assert idx[0] == 0 and np.isnan(mx[0])
    # bf16 inf in the activation: rows with positive weight -> +inf, others NaN/-inf
    hi = synth.f32_to_bf16_bits(np.array([[np.inf] + [0.0] * (k - 1)], np.float32))
    codes = np.zeros((4, k // 2), np.uint8)
    codes[1, 0] = 0x02          # +1.0 at k=0 -> +inf
    codes[2, 0] = 0x0A          # -1.0 at k=0 -> -inf
    codes[3, 0] = 0x02          # +inf again, later index
    idx, mx = orc.lmhead_argmax(hi, codes, scales, np.float32(1.0))
    assert idx[0] == 1 and mx[0] == np.inf
    # signed zeros: every logit is +-0, index 0 wins
    hz = synth.f32_to_bf16_bits(np.zeros((1, k), np.float32))
    codes = np.full((4, k // 2), 0x99, np.uint8)
    idx, mx = orc.lmhead_argmax(hz, codes, scales, np.float32(1.0))
    assert idx[0] == 0
