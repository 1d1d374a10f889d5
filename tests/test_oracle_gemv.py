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

from nvfp4_w4a16_mtp_amd import synth

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
