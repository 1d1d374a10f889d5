"""Pins for the oracle's codecs (CPU only).

The E2M1 and E4M3FN formats are the public OCP FP4/FP8 definitions (the
pages name NVFP4 only through the quantizer kernels that new.rs resolves in
`MtpHead::new`).  Each test compares the oracle with something other than
itself: printed format facts, torch's own float8_e4m3fn / bfloat16 casts, or
brute-force nearest-point searches over every input in a range.
"""
import numpy as np
import pytest
import torch

# E2M1 magnitudes as the OCP FP4 spec tabulates them (codes 0..7).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_table(orc):
    for c in range(16):
        want = E2M1_TABLE[c & 7] * (-1.0 if c & 8 else 1.0)
        got = orc.e2m1_decode(c)
        assert got == want and np.signbit(got) == bool(c & 8)


def test_e2m1_roundtrip(orc):
    for c in range(16):
        assert orc.e2m1_encode(orc.e2m1_decode(c)) == c


def _brute_e2m1(v: np.ndarray) -> np.ndarray:
    """Independent nearest-grid-point search: locate |v| between its two grid
    neighbours, take the nearer, on a tie take the even code; saturate at 6;
    the sign bit is copied from v."""
    grid = np.array(E2M1_TABLE)
    a = np.abs(v.astype(np.float64))
    idx = np.searchsorted(grid, a)                 # grid[idx-1] < a <= grid[idx]
    hi = np.clip(idx, 0, 7)
    lo = np.clip(idx - 1, 0, 7)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick = np.where(dlo < dhi, lo, hi)
    tie = (dlo == dhi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a >= 6.0, 7, pick)
    return (pick | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


@pytest.mark.parametrize("exp", list(range(-3, 3)))
def test_e2m1_encode_exhaustive_binade(orc, exp):
    """Every fp32 with |v| in [2^exp, 2^(exp+1)), both signs: covers every
    rounding threshold (0.25 .. 5) and the saturation boundary at 6..8."""
    base = np.float32(2.0 ** exp).view(np.uint32)
    bits = (base + np.arange(1 << 23, dtype=np.uint32)).astype(np.uint32)
    for sign in (0, 0x80000000):
        v = (bits | np.uint32(sign)).view(np.float32)
        assert np.array_equal(orc.e2m1_encode_array(v), _brute_e2m1(v))


def test_e2m1_encode_extremes(orc):
    tiny = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-20, 0.1249, -0.1249], np.float32)
    assert np.array_equal(orc.e2m1_encode_array(tiny), _brute_e2m1(tiny))
    big = np.array([8.0, 1e30, np.inf, -8.0, -np.inf, 3.4e38], np.float32)
    assert list(orc.e2m1_encode_array(big)) == [7, 7, 7, 15, 15, 7]


def test_e4m3_decode_vs_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        got = orc.e4m3_decode(b)
        if np.isnan(ref[b]):
            assert np.isnan(got) and (b & 0x7F) == 0x7F
        else:
            assert got == ref[b]


def test_e4m3_printed_facts(orc):
    assert orc.e4m3_decode(0x7E) == 448.0          # largest finite
    assert orc.e4m3_decode(0x08) == 2.0 ** -6      # smallest normal
    assert orc.e4m3_decode(0x01) == 2.0 ** -9      # smallest subnormal
    assert orc.e4m3_decode(0x38) == 1.0
    vals = [orc.e4m3_decode(b) for b in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))   # strictly increasing


def test_e4m3_roundtrip(orc):
    for b in range(0x7F):
        assert orc.e4m3_encode(orc.e4m3_decode(b)) == b


def _grid_e4m3():
    return torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


@pytest.mark.parametrize("exp", [-12, -11, -10, -9, -8, -7, -6, -5, 0, 7, 8])
def test_e4m3_encode_exhaustive_binade(orc, exp):
    """Every fp32 in [2^exp, 2^(exp+1)): nearest of the 127 non-negative grid
    points, ties to the even byte (= even mantissa), saturating to 0x7E.  The
    binades cover everything below the smallest subnormal, the subnormal
    range and its hand-over to the normals, one ordinary binade, and the top
    two (448 and saturation)."""
    grid = _grid_e4m3()
    base = np.float32(2.0 ** exp).view(np.uint32)
    bits = (base + np.arange(1 << 23, dtype=np.uint32)).astype(np.uint32)
    s = bits.view(np.float32)
    got = orc.e4m3_encode_array(s)
    idx = np.searchsorted(grid, s.astype(np.float64))      # grid[idx-1] < s <= grid[idx]
    idx_hi = np.clip(idx, 0, 126)
    idx_lo = np.clip(idx - 1, 0, 126)
    dlo = np.abs(s - grid[idx_lo])
    dhi = np.abs(grid[idx_hi] - s)
    want = np.where(dlo < dhi, idx_lo, idx_hi)
    tie = (dlo == dhi) & (idx_lo != idx_hi)
    want = np.where(tie, np.where(idx_lo % 2 == 0, idx_lo, idx_hi), want)
    want = np.where(s >= 448.0, 126, want)
    assert np.array_equal(got, want.astype(np.uint8))


def test_e4m3_encode_small_and_large(orc):
    s = np.array([0.0, 1e-45, 1e-30, 2.0 ** -13, 448.0, 463.9, 464.0, 1e6, 3e38, np.inf], np.float32)
    assert list(orc.e4m3_encode_array(s)) == [0, 0, 0, 0, 126, 126, 126, 126, 126, 126]


def test_e4m3_encode_vs_torch_cast(orc):
    """torch's float32 -> float8_e4m3fn cast is round-to-nearest-even; it
    agrees with saturation on [0, 464], where it still returns 448."""
    rng = np.random.default_rng(0)
    s = np.concatenate([rng.uniform(0, 464, 200000), 2.0 ** rng.uniform(-12, 8.8, 200000)])
    s = s[s <= 464].astype(np.float32)
    ref = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode_array(s), ref)


def test_bf16_round_vs_torch(orc):
    rng = np.random.default_rng(1)
    v = rng.standard_normal(5000).astype(np.float32) * np.float32(3.0)
    # include exact ties (low 16 bits == 0x8000)
    ties = (rng.integers(0, 1 << 16, 2000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    for arr in (v, ties):
        ref = torch.from_numpy(arr).to(torch.bfloat16).float().numpy()
        got = np.array([orc.bf16_round(float(a)) for a in arr], np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
