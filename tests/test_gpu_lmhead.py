"""GPU parity: lmhead_gemv_argmax (C ABI) vs the oracle.  The index must be
bit-exact: on planted inputs the winner is certified by a closed-form margin
far above the fp32 rounding bound; on random inputs a row is compared only
when the oracle's top-2 gap exceeds the rigorous bound, otherwise the GPU's
index must be one whose logit is within the bound of the maximum."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _gpu(h, wd, vrows=0, bf16=False):
    import nvfp4_w4a16_mtp_amd as nv
    idx, mx = nv.lmhead_gemv_argmax(dev_bf16(h), wd, vocab_rows=vrows, bf16_keys=bf16)
    return idx.cpu().numpy(), mx.cpu().numpy()


def _check_certified(orc, h, codes, scales, g, vrows=0):
    """Compare with the oracle; rows whose winner is not certified accept any
    index whose logit lies within the error bound of the maximum."""
    idx, mx = _gpu(h, _w(codes, scales, g), vrows)
    ridx, rmx, logits, absb = orc.lmhead_argmax(h, codes, scales, g, vrows=vrows, want_logits=True)
    k = h.shape[1]
    gamma = (k + 8) * 2.0 ** -24                      # fp32 accumulation bound factor
    for i in range(h.shape[0]):
        bound = gamma * absb[i] + 1e-30
        top = logits[i, ridx[i]]
        others = np.delete(np.arange(logits.shape[1]), ridx[i])
        # rows identical to the winner have identical logits on both sides
        same = (codes[others] == codes[ridx[i]]).all(axis=1) & (scales[others] == scales[ridx[i]]).all(axis=1)
        gap_ok = (top - logits[i, others] > bound[ridx[i]] + bound[others]) | same
        if gap_ok.all():
            assert idx[i] == ridx[i], (i, idx[i], ridx[i])
        else:
            assert logits[i, idx[i]] >= top - bound[ridx[i]] - bound[idx[i]], (i, idx[i], ridx[i])
        assert_close(mx[i:i + 1], logits[i, idx[i]:idx[i] + 1], "max logit")
    return idx, ridx


def test_tiny_planted(orc):
    w = synth.weight_bf16(0, 4096, 256)
    h = synth.acts_bf16(0, 1, 256)
    codes, scales, glob = orc.quantize(w)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=0, n_near=4, dup=True)
    idx, ridx = _check_certified(orc, h, codes, scales, glob[0])
    assert idx[0] == min([info["star"][0]] + info["dups"][0])


@pytest.mark.parametrize("m", list(range(1, 9)))
def test_random_unplanted(orc, m):
    w = synth.weight_bf16(50 + m, 3000, 512)
    h = synth.acts_bf16(50 + m, m, 512)
    codes, scales, glob = orc.quantize(w)
    _check_certified(orc, h, codes, scales, glob[0])


@pytest.mark.parametrize("m,v,k", [(5, 3001, 1024), (7, 1000, 3072), (8, 17, 2048), (6, 4096, 7168), (4, 999, 2048),
                                   (8, 700, 9216)])
def test_random_unplanted_eight_row_units(orc, m, v, k):
    """Four to eight rows with K a multiple of 1024 (16-row MFMA units):
    ragged vocabularies, rows padded; at K = 9216 eight rows and the staging
    areas exceed the LDS and the dot2 units serve them."""
    w = synth.weight_bf16(60 + m, v, k)
    h = synth.acts_bf16(60 + m, m, k)
    codes, scales, glob = orc.quantize(w)
    _check_certified(orc, h, codes, scales, glob[0])


@pytest.mark.parametrize("vocab", [32768, 151936])
@pytest.mark.parametrize("m", [1, 4, 8])
def test_config_planted_near_ties(orc, vocab, m):
    """Full vocabulary weight [151936, 2048]; V = 32768 scores the prefix."""
    codes, scales, glob = _full_head(orc)
    codes, scales = codes.copy(), scales.copy()
    h = synth.acts_bf16(60 + m, m, 2048)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=60 + m, n_near=4, dup=(m % 2 == 0), vrows=vocab)
    idx, ridx = _check_certified(orc, h, codes, scales, glob[0], vrows=vocab)
    for i in range(m):
        assert idx[i] == min([info["star"][i]] + info["dups"][i])


_HEAD = {}


def _full_head(orc):
    if "q" not in _HEAD:
        w = synth.weight_bf16(77, 151936, 2048)
        import nvfp4_w4a16_mtp_amd as nv
        q = nv.nvfp4_quantize(dev_bf16(w))
        codes, scales, glob = orc.quantize(w)
        # the full LM head is also the largest quantizer parity case
        assert np.array_equal(q.scales.cpu().numpy(), scales)
        assert np.array_equal(q.codes.cpu().numpy(), codes)
        _HEAD["q"] = (codes, scales, glob)
    return _HEAD["q"]


def test_duplicates_lowest_index(orc):
    """Exact copies of the winning row resolve to the lowest copy, also in
    bf16-key mode where many rows share the maximum key."""
    x, codes, scales, g = synth.exact_family(5, 3, 5000, 256)
    codes[4321] = codes[17]
    scales[4321] = scales[17]
    codes[123] = codes[17]
    scales[123] = scales[17]
    for bf16 in (False, True):
        idx, mx = _gpu(x, _w(codes, scales, g), bf16=bf16)
        ridx, rmx = orc.lmhead_argmax(x, codes, scales, g, flags=int(bf16))
        assert np.array_equal(idx, ridx) and np.array_equal(mx, rmx)


@pytest.mark.parametrize("vrows", [1, 2, 17, 4095, 4096, 0, 10 ** 6])
def test_reduced_vocab_exact(orc, vrows):
    x, codes, scales, g = synth.exact_family(6, 8, 4096, 512)
    idx, mx = _gpu(x, _w(codes, scales, g), vrows)
    ridx, rmx = orc.lmhead_argmax(x, codes, scales, g, vrows=vrows)
    assert np.array_equal(idx, ridx) and np.array_equal(mx.view(np.uint32), rmx.view(np.uint32))


def test_nonfinite(orc):
    k = 32
    scales = np.full((4, 2), 0x38, np.uint8)
    codes = np.full((4, 16), 0x11, np.uint8)
    h = synth.f32_to_bf16_bits(np.ones((1, k), np.float32))
    idx, mx = _gpu(h, _w(codes, scales, np.nan))
    assert idx[0] == 0 and np.isnan(mx[0])
    hi = synth.f32_to_bf16_bits(np.array([[np.inf] + [0.0] * (k - 1)], np.float32))
    codes = np.zeros((4, 16), np.uint8)
    codes[1, 0] = 0x02
    codes[2, 0] = 0x0A
    codes[3, 0] = 0x02
    idx, mx = _gpu(hi, _w(codes, scales, 1.0))
    ridx, rmx = orc.lmhead_argmax(hi, codes, scales, np.float32(1.0))
    assert idx[0] == ridx[0] == 1 and mx[0] == np.inf
