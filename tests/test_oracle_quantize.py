"""Pins for the oracle's NVFP4 quantizer (CPU only).

The quantizer is the two-pass scheme new.rs resolves in `MtpHead::new`
(global absmax, then per-block scales and codes).  The pins: a hand-worked
golden row, invariants every correct quantization satisfies, and
metamorphic relations (power-of-two scaling, negation).
"""
import json
import os

import numpy as np
import pytest
import torch

from tests import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_block.json")
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _unpack(codes):
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def _e2m1_val(code):
    v = E2M1_TABLE[code & 7]
    return np.where(code & 8, -v, v)


def test_worked_block(orc):
    g = json.load(open(GOLDEN))
    row = np.array(g["row"], np.float32)[None, :]
    w = synth.f32_to_bf16_bits(row)
    assert np.array_equal(synth.bf16_bits_to_f32(w), row)    # the row is exact in bf16
    codes, scales, glob = orc.quantize(w)
    assert list(_unpack(codes)[0]) == g["codes"]
    assert list(scales[0]) == g["scales"]
    assert glob[0] == g["g_dec"] and glob[1] == g["g_enc"] and glob[2] == g["amax"]


def test_global_scales(orc):
    w = synth.weight_bf16(3, 64, 128)
    f = synth.bf16_bits_to_f32(w)
    amax = np.abs(f).max()
    g_dec, g_enc, a = orc.global_scales(w)
    assert a == amax
    assert g_enc == np.float32(2688.0) / np.float32(amax)
    assert g_dec == np.float32(amax) / np.float32(2688.0)
    assert abs(float(g_dec) * float(g_enc) - 1.0) <= 2.0 ** -22


def test_zero_tensor(orc):
    w = np.zeros((4, 32), np.uint16)
    codes, scales, glob = orc.quantize(w)
    assert not codes.any() and not scales.any() and not glob.any()
    wneg = np.full((4, 32), 0x8000, np.uint16)   # all -0.0
    codes, scales, glob = orc.quantize(wneg)
    assert (codes == 0x88).all() and not scales.any()


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_invariants(orc, seed):
    n, k = 48, 256
    w = synth.weight_bf16(seed, n, k)
    if seed == 4:     # heavy-tailed rows with many tiny blocks: exercises subnormal scales
        f = synth.bf16_bits_to_f32(w) * np.float32(10.0) ** np.random.default_rng(9).uniform(-4, 0, (n, 1)).astype(np.float32)
        w = synth.f32_to_bf16_bits(f)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    codes, scales, glob = orc.quantize(w)
    g_dec = float(glob[0])
    sf = _e4m3_table()[scales]                                    # [n, k/16]
    assert (scales <= 0x7E).all()
    c = _unpack(codes)
    what = _e2m1_val(c) * np.repeat(sf, 16, axis=1) * g_dec
    # (i) the dequantized value set equals the oracle's own dequantizer
    assert np.array_equal(what, orc.dequantize(codes, scales, glob[0], n, k))
    # (ii) the block maximum maps to the top code wherever the scale is normal
    blk = np.abs(wf).reshape(n, k // 16, 16)
    arg = blk.argmax(axis=2)
    cb = c.reshape(n, k // 16, 16)
    top = np.take_along_axis(cb, arg[..., None], axis=2)[..., 0] & 7
    normal = (scales >= 0x08) & (blk.max(axis=2) > 0)
    assert (top[normal] >= 6).all()
    big = normal & (scales >= 0x10)
    assert (top[big] == 7).all()
    # (iii) per-element error within half the local grid gap (plus fp32 slack)
    a = np.abs(wf) * float(glob[1]) / np.repeat(np.maximum(sf, 1e-30), 16, axis=1)
    gap = np.where(a <= 2, 0.5, np.where(a <= 4, 1.0, 2.0))
    err = np.abs(wf - what)
    lim = 0.5 * gap * np.repeat(sf, 16, axis=1) * g_dec * (1 + 1e-5) + 1e-30
    sat = a > 6
    assert (err[~sat] <= lim[~sat]).all()


@pytest.mark.parametrize("j", [-20, -3, 1, 7])
def test_power_of_two_scaling(orc, j):
    w = synth.weight_bf16(5, 32, 128)
    w2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(w) * np.float32(2.0 ** j))
    c1, s1, g1 = orc.quantize(w)
    c2, s2, g2 = orc.quantize(w2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert g2[0] == np.float32(g1[0] * 2.0 ** j)
    assert g2[2] == np.float32(g1[2] * 2.0 ** j)


def test_negation_flips_sign_bits(orc):
    w = synth.weight_bf16(6, 32, 128)
    c1, s1, g1 = orc.quantize(w)
    c2, s2, g2 = orc.quantize(w ^ np.uint16(0x8000))
    assert np.array_equal(c1 ^ 0x88, c2) and np.array_equal(s1, s2) and np.array_equal(g1, g2)


def test_extreme_magnitudes(orc):
    """Largest bf16 magnitudes and tiny tensors stay finite and well formed."""
    for scale in (3.0e38, 1e-30, 1e-36):
        w = synth.f32_to_bf16_bits(np.linspace(-1, 1, 64 * 32).astype(np.float32).reshape(64, 32) * np.float32(scale))
        codes, scales, glob = orc.quantize(w)
        assert np.isfinite(glob).all() and (scales <= 0x7E).all()
        assert (_unpack(codes)[np.abs(synth.bf16_bits_to_f32(w)) == np.abs(synth.bf16_bits_to_f32(w)).max()] & 7 == 7).all()
