"""Pins for the oracle's W4A16 GEMV / GEMM (CPU only).

`y[m, n] = sum_k x[m, k] * W^[n, k]` is the `out = in @ W^T` convention of
mtp_head.rs (`MtpHead::gemv`) and of the prefill GEMM in prefill_weights.rs
(`w4a16_gemm_m128_dispatch`).  Pins: exact rational arithmetic on tiny
shapes, a textbook matvec special case, the exact-arithmetic family, and
GEMM-with-M-rows = M separate GEMVs.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests import synth

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _frac_weight(codes, scales, g_dec, n, k):
    out = []
    for r in range(n):
        row = []
        for c in range(k):
            byte = int(codes[r, c // 2])
            code = (byte >> 4) if c & 1 else (byte & 15)
            v = Fraction(E2M1[code & 7]) * (-1 if code & 8 else 1)
            row.append(v * Fraction(float(E4M3[scales[r, c // 16]])) * Fraction(float(g_dec)))
        out.append(row)
    return out


def _ulp32(v: float) -> float:
    v = np.float32(abs(v))
    return float(np.nextafter(v, np.float32(np.inf)) - v) if v != 0 else float(np.float32(1e-45))


@pytest.mark.parametrize("seed,m,n,k", [(0, 1, 8, 32), (1, 4, 32, 64), (2, 3, 17, 32), (3, 2, 5, 64)])
def test_exact_rationals(orc, seed, m, n, k):
    w = synth.weight_bf16(seed, n, k)
    x = synth.acts_bf16(seed, m, k)
    codes, scales, glob = orc.quantize(w)
    y = orc.gemv(x, codes, scales, glob[0])
    W = _frac_weight(codes, scales, glob[0], n, k)
    xf = synth.bf16_bits_to_f32(x)
    for i in range(m):
        X = [Fraction(float(v)) for v in xf[i]]
        for r in range(n):
            exact = sum(a * b for a, b in zip(X, W[r]))
            want = np.float32(float(exact))             # fl32 of the exact value (<=1 ulp double rounding)
            assert abs(float(y[i, r]) - float(want)) <= _ulp32(float(want)), (i, r)


def test_unit_scale_is_textbook_matvec(orc):
    """With every block scale 1.0 (0x38) and g_dec = 1, W^ is a plain matrix
    of E2M1 values and the GEMV is numpy's matvec in float64."""
    rng = np.random.default_rng(7)
    n, k = 40, 96
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = np.full((n, k // 16), 0x38, np.uint8)
    x = synth.acts_bf16(7, 3, k)
    lo, hi = codes & 15, codes >> 4
    cw = np.empty((n, k), np.int64)
    cw[:, 0::2], cw[:, 1::2] = lo, hi
    Wv = np.array(E2M1)[cw & 7] * np.where(cw & 8, -1.0, 1.0)
    ref = (synth.bf16_bits_to_f32(x).astype(np.float64) @ Wv.T).astype(np.float32)
    got = orc.gemv(x, codes, scales, np.float32(1.0))
    assert np.array_equal(got, ref)


def test_exact_family_is_exact(orc):
    x, codes, scales, g_dec = synth.exact_family(11, 4, 64, 4096)
    y = orc.gemv(x, codes, scales, g_dec)
    Wv = np.array([[float(v) for v in row] for row in _frac_weight(codes[:3], scales[:3], g_dec, 3, 4096)])
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ Wv.T
    assert np.array_equal(y[:, :3].astype(np.float64), ref)
    # every value is a multiple of g_dec/8 below 2^21 * g_dec
    q = y.astype(np.float64) / (float(g_dec) / 8)
    assert np.array_equal(q, np.round(q)) and (np.abs(y) < 2.0 ** 21 * float(g_dec)).all()


def test_gemm_rows_equal_gemv(orc):
    w = synth.weight_bf16(12, 24, 128)
    x = synth.acts_bf16(12, 9, 128)
    codes, scales, glob = orc.quantize(w)
    full = orc.gemv(x, codes, scales, glob[0])
    for i in range(9):
        assert np.array_equal(full[i:i + 1], orc.gemv(x[i:i + 1], codes, scales, glob[0]))
    mi = np.array([0, 3, 8, 5], np.int64)
    ni = np.array([23, 0, 7, 11], np.int64)
    assert np.array_equal(orc.gemm_sample(x, codes, scales, glob[0], mi, ni), full[mi, ni])


def test_dequantize_matches_library_decode(orc):
    w = synth.weight_bf16(13, 16, 64)
    codes, scales, glob = orc.quantize(w)
    W = np.array([[float(v) for v in row] for row in _frac_weight(codes, scales, glob[0], 16, 64)])
    assert np.array_equal(orc.dequantize(codes, scales, glob[0], 16, 64), W)


def test_scale_range_family_is_exact(orc):
    """The scale-range family (every E4M3 byte, zero and subnormal scales,
    negative scales) has exact dot products: the oracle's fp32 result equals
    the exact rational sum, and fp32 accumulation in a shuffled order of
    block partials (the GPU's kind of order) gives the same bits."""
    x, codes, scales, g_dec = synth.scale_range_family(12, 2, 32, 512)
    assert sorted(set((scales & 0x7F).ravel().tolist())) == list(range(127))
    y = orc.gemv(x, codes, scales, g_dec)
    W = _frac_weight(codes, scales, g_dec, 32, 512)
    xf = synth.bf16_bits_to_f32(x)
    rng = np.random.default_rng(12)
    for i in range(2):
        X = [Fraction(float(v)) for v in xf[i]]
        for r in range(32):
            exact = sum(a * b for a, b in zip(X, W[r]))
            assert Fraction(float(y[i, r])) == exact, (i, r)
            terms = np.array([float(a * b) for a, b in zip(X, W[r])], np.float32)
            blocks = [np.float32(0)] * 32
            for b in range(32):
                s = np.float32(0)
                for t in terms[16 * b:16 * b + 16]:
                    s = np.float32(s + t)
                blocks[b] = s
            acc = np.float32(0)
            for b in rng.permutation(32):
                acc = np.float32(acc + blocks[b])
            assert acc == np.float32(y[i, r]), (i, r)


def test_scale_range_worst_case_under_2_24_quanta():
    """The bound behind the family's exactness at K = 17408: in every binade
    window the largest |x * e2m1 * scale| sum over a row stays below 2^24
    quanta of half the window's scale quantum."""
    for j in range(16):
        lo, hi = 8 * j, min(8 * j + 7, 0x7E)
        vals = [float(E4M3[b]) for b in range(lo, hi + 1)]
        quantum = 2.0 ** -9 if j <= 1 else 2.0 ** (j - 10)
        assert all(v / quantum == round(v / quantum) for v in vals)
        worst = 17408 * 3 * 6 * max(vals)                 # |x| <= 3, |e2m1| <= 6
        assert worst / (quantum / 2) < 2.0 ** 24, j


def test_decode_rows_closed_form(orc):
    """One row per E4M3 byte with codes 1.0 and one-hot activations: the
    oracle gives g_dec * e4m3(byte) * sum(x) (the table of torch's float8)."""
    x, codes, scales, byt = synth.scale_decode_rows(3, 256, seed=5)
    y = orc.gemv(x, codes, scales, np.float32(0.5))
    xs = synth.bf16_bits_to_f32(x).astype(np.float64).sum(axis=1)
    assert np.array_equal(y, (0.5 * xs[:, None] * E4M3[byt][None, :]).astype(np.float32))
    assert byt.size == 254 and 0x7F not in byt and 0xFF not in byt


def test_thread_count_does_not_change_results(orc):
    """The oracle splits independent outputs over threads; one thread and
    every thread give the same bits (GEMV, LM-head argmax and logits, MoE,
    quantizer)."""
    w = synth.weight_bf16(14, 300, 512)
    x = synth.acts_bf16(14, 3, 512)
    ex = synth.moe_quantized_experts(14, 16, 256, 128)
    xm = synth.acts_bf16(15, 2, 256)
    r = synth.router_logits(15, 2, 16)
    n0 = orc.get_threads()
    outs = []
    for n in (1, max(2, n0)):
        orc.set_threads(n)
        c, s, g = orc.quantize(w)
        outs.append((c, s, orc.gemv(x, c, s, g[0]), *orc.lmhead_argmax(x, c, s, g[0], want_logits=True),
                     *orc.moe(xm, r, 4, *ex)))
    orc.set_threads(n0)
    for a, b in zip(*outs):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
