"""GPU parity: w4a16_gemv (C ABI) vs the oracle.  Bit-exact on the exact-
arithmetic family, within |d| <= 1e-3 + 2e-3 |ref| on normal inputs, at the
tiny and the Qwen-shaped projection sizes for M = 1..8."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, bf16_round_f64, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu

PROJ = {"fc": (2048, 4096), "q": (8192, 2048), "k": (512, 2048), "v": (512, 2048), "o": (2048, 4096)}


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


@pytest.mark.parametrize("m", range(1, 9))
@pytest.mark.parametrize("n,k", [(64, 32), (333, 512), (96, 4096), (2050, 2048)])
def test_exact_family_bit_exact(orc, m, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(100 + m, m, n, k)
    y = nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def test_tiny_config(orc):
    import nvfp4_w4a16_mtp_amd as nv
    w = synth.weight_bf16(0, 512, 256)
    x = synth.acts_bf16(0, 1, 256)
    q = nv.nvfp4_quantize(dev_bf16(w))
    codes, scales, glob = orc.quantize(w)
    assert np.array_equal(q.codes.cpu().numpy(), codes)
    y = nv.w4a16_gemv(dev_bf16(x), q).cpu().numpy()
    assert_close(y, orc.gemv(x, codes, scales, glob[0]), "tiny")


@pytest.mark.parametrize("name", list(PROJ))
@pytest.mark.parametrize("m", [1, 4, 8])
def test_projection_configs(orc, name, m):
    import nvfp4_w4a16_mtp_amd as nv
    n, k = PROJ[name]
    w = synth.weight_bf16(20 + len(name), n, k)
    x = synth.acts_bf16(30 + m, m, k)
    codes, scales, glob = orc.quantize(w)
    y = nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, glob[0])).cpu().numpy()
    assert_close(y, orc.gemv(x, codes, scales, glob[0]), f"{name} m={m}")


@pytest.mark.parametrize("m", [1, 3, 8])
def test_bf16_output(orc, m):
    import nvfp4_w4a16_mtp_amd as nv
    w = synth.weight_bf16(40, 700, 1024)
    x = synth.acts_bf16(41, m, 1024)
    codes, scales, glob = orc.quantize(w)
    wd = _w(codes, scales, glob[0])
    y32 = nv.w4a16_gemv(dev_bf16(x), wd).cpu().numpy()
    yb = nv.w4a16_gemv(dev_bf16(x), wd, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(yb, bf16_round_f64(y32).astype(np.float32))      # RNE of the fp32 result
    ref = orc.gemv(x, codes, scales, glob[0])
    ulp = np.abs(bf16_round_f64(ref)) * 2.0 ** -7
    assert (np.abs(yb - bf16_round_f64(ref)) <= ulp + 1e-30).all()           # within 1 bf16 ulp


def test_empty_and_errors():
    import nvfp4_w4a16_mtp_amd as nv
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    w0 = nv.NVFP4Weight.from_parts(torch.zeros((0, 32), dtype=torch.uint8, device="cuda"),
                                   torch.zeros((0, 4), dtype=torch.uint8, device="cuda"), 1.0)
    assert nv.w4a16_gemv(x, w0).shape == (1, 0)
    w = nv.NVFP4Weight.from_parts(torch.zeros((4, 32), dtype=torch.uint8, device="cuda"),
                                  torch.zeros((4, 4), dtype=torch.uint8, device="cuda"), 1.0)
    with pytest.raises(nv.NVFP4Error):
        nv.w4a16_gemv(torch.zeros((9, 64), dtype=torch.bfloat16, device="cuda"), w)
    bad = nv.NVFP4Weight(w.codes, w.scales, w.glob, 4, 48)
    with pytest.raises(nv.NVFP4Error):
        nv.w4a16_gemv(torch.zeros((1, 48), dtype=torch.bfloat16, device="cuda"), bad)


def test_no_write_outside_output(orc):
    """Canary words around y stay untouched."""
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(7, 3, 100, 256)
    buf = torch.full((3 * 100 + 128,), 12345.0, dtype=torch.float32, device="cuda")
    y = buf[64:64 + 300].view(3, 100)
    nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, g), out=y)
    b = buf.cpu().numpy()
    assert (b[:64] == 12345.0).all() and (b[364:] == 12345.0).all()
    assert np.array_equal(y.cpu().numpy(), orc.gemv(x, codes, scales, g))


# Weights with enough units for the persistent streaming grid on a 256-CU
# MI355X (two units per wavefront at one or two rows; the MFMA units at five
# to eight rows), ragged row counts; the exact family makes every output bit
# exact in any summation order.
@pytest.mark.parametrize("m,n,k", [(1, 16387, 2048), (1, 32771, 512), (2, 49155, 256), (8, 8195, 1024),
                                   (6, 20000, 2048), (4, 8195, 1024), (8, 8195, 9216)])
def test_persistent_grid_bit_exact(orc, m, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(150 + m, m, n, k)
    y = nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


# Few row tiles and K a multiple of 512 per wavefront slice with a chunk
# count outside 1, 2, 4 (5, 7, 3, 6, 17 a lane): the K split of the
# pipelined generic loop, with a partial last stage, ragged row counts.
@pytest.mark.parametrize("m,n,k", [(1, 333, 5120), (2, 200, 7168), (4, 90, 3072), (1, 100, 12288),
                                   (1, 1041, 17408), (2, 1040, 5120)])
def test_k_split_pipelined_bit_exact(orc, m, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(170 + m, m, n, k)
    y = nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


# Activation images of a quarter of a CU's LDS or more: wide workgroups
# (8 or 16 wavefronts, the K of 16 rows split over 2 or 4 wavefront groups),
# K slices whose chunk counts differ between the lanes (17408 / 32 / 4 = 136
# chunks over 16 lanes), ragged row counts.
@pytest.mark.parametrize("m,n,k", [(2, 700, 17408), (4, 333, 17408), (3, 300, 10240), (8, 120, 5120),
                                   (2, 90, 12288), (4, 17, 9728)])
def test_wide_workgroups_bit_exact(orc, m, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(190 + m, m, n, k)
    y = nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m,n,k", [(5, 300, 10240), (8, 301, 17408), (3, 77, 40960)])
def test_rows_beyond_the_lds_go_in_groups(orc, m, n, k):
    """round_up(m) rows of K do not fit the LDS image: the rows go in groups
    (5 -> 4 + 1, 8 -> 4 + 4, 3 -> 1 + 1 + 1); the bf16 output is the
    rounding of the fp32 one, and odd n puts bf16 groups at 2-byte offsets."""
    import nvfp4_w4a16_mtp_amd as nv
    w = synth.weight_bf16(160 + m, n, k)
    x = synth.acts_bf16(161 + m, m, k)
    codes, scales, glob = orc.quantize(w)
    wd = _w(codes, scales, glob[0])
    y32 = nv.w4a16_gemv(dev_bf16(x), wd).cpu().numpy()
    assert_close(y32, orc.gemv(x, codes, scales, glob[0]), f"m={m} k={k}")
    yb = nv.w4a16_gemv(dev_bf16(x), wd, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(yb, bf16_round_f64(y32).astype(np.float32))


# Four to eight activation rows, K a whole number of 1024-wide slices (1 to
# 8), few enough 16-row units: the K-split MFMA units (one wavefront per
# slice, the slices' sums added in slice order), ragged row counts, both
# families, fp32 and bf16 outputs.
@pytest.mark.parametrize("m,n,k", [(3, 17, 1024), (4, 333, 3072), (5, 700, 5120), (8, 2050, 7168), (6, 95, 8192),
                                   (8, 16383, 2048), (4, 40000, 1024)])
@pytest.mark.parametrize("fam", ["exact", "scales"])
def test_mfma_k_split_bit_exact(orc, m, n, k, fam):
    import nvfp4_w4a16_mtp_amd as nv
    gen = synth.exact_family if fam == "exact" else synth.scale_range_family
    x, codes, scales, g = gen(230 + m + n, m, n, k)
    wd = _w(codes, scales, g)
    ref = orc.gemv(x, codes, scales, g)
    y = nv.w4a16_gemv(dev_bf16(x), wd).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
    yb = nv.w4a16_gemv(dev_bf16(x), wd, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(yb, bf16_round_f64(ref).astype(np.float32))


@pytest.mark.parametrize("m", [4, 7, 8])
def test_mfma_k_split_grouped_with_empty_groups(orc, m):
    import nvfp4_w4a16_mtp_amd as nv
    parts = [synth.exact_family(240 + 5 * i + m, m, n, 4096) for i, n in enumerate((0, 511, 0, 33, 1))]
    x = parts[1][0]
    ws = [_w(c, s, g) for _, c, s, g in parts]
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), ws)
    for (_, c, s, g), y in zip(parts, ys):
        if c.shape[0]:
            assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.gemv(x, c, s, g).view(np.uint32))
