"""GPU parity: nvfp4_quantize (C ABI) vs the oracle, bit-exact on codes,
scales and the global struct."""
import json
import os

import numpy as np
import pytest

from tests import synth
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def _run(w_bits):
    import nvfp4_w4a16_mtp_amd as nv
    q = nv.nvfp4_quantize(dev_bf16(w_bits))
    return q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.glob.cpu().numpy()


def _check(orc, w_bits):
    c, s, g = _run(w_bits)
    rc, rs, rg = orc.quantize(w_bits)
    assert np.array_equal(s, rs), "scales differ"
    assert np.array_equal(c, rc), "codes differ"
    assert g[0].view(np.uint32) == rg[0].view(np.uint32) and g[1].view(np.uint32) == rg[1].view(np.uint32)
    assert g[2] == rg[2] and g[3].view(np.uint32) == 0


def test_worked_block(orc):
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_block.json")))
    w = synth.f32_to_bf16_bits(np.array(gold["row"], np.float32)[None, :])
    c, s, g = _run(w)
    lo, hi = c[0] & 15, c[0] >> 4
    codes = np.empty(32, np.uint8)
    codes[0::2], codes[1::2] = lo, hi
    assert list(codes) == gold["codes"] and list(s[0]) == gold["scales"]
    assert g[0] == gold["g_dec"] and g[1] == gold["g_enc"] and g[2] == gold["amax"]


@pytest.mark.parametrize("seed,n,k", [(0, 512, 256), (1, 37, 96), (2, 1, 32), (3, 300, 2048)])
def test_random(orc, seed, n, k):
    _check(orc, synth.weight_bf16(seed, n, k))


@pytest.mark.parametrize("scale", [3.0e38, 1e-30, 1e-36, 2.0 ** -120, 1.0])
def test_magnitudes(orc, scale):
    w = synth.bf16_bits_to_f32(synth.weight_bf16(7, 64, 128)) * np.float32(scale / 0.02)
    _check(orc, synth.f32_to_bf16_bits(w))


def test_heavy_tailed_rows_subnormal_scales(orc):
    f = synth.bf16_bits_to_f32(synth.weight_bf16(8, 96, 256))
    f = f * np.float32(10.0) ** np.random.default_rng(8).uniform(-5, 0, (96, 1)).astype(np.float32)
    _check(orc, synth.f32_to_bf16_bits(f))


def test_zero_and_signed_zero(orc):
    _check(orc, np.zeros((8, 64), np.uint16))
    _check(orc, np.full((8, 64), 0x8000, np.uint16))


def test_tie_points(orc):
    """Every E2M1 tie point hit exactly (scale 1, g_enc 1) in every position."""
    rng = np.random.default_rng(9)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, 0.5], np.float32)
    f = rng.choice(ties, size=(64, 128)) * rng.choice([-1.0, 1.0], size=(64, 128)).astype(np.float32)
    f[:, ::16] = 6.0          # every block max 6 -> scale exactly 1
    f[0, 0] = 2688.0          # tensor max -> g_enc exactly 1
    _check(orc, synth.f32_to_bf16_bits(f))


@pytest.mark.parametrize("shape", [(8192, 2048), (2048, 4096)])
def test_projection_shapes(orc, shape):
    _check(orc, synth.weight_bf16(10, *shape))
