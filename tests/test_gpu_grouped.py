"""GPU parity: w4a16_gemv_grouped (C ABI) vs the oracle's GEMV applied to
each weight.  Bit-exact on the exact-arithmetic family; within
|d| <= 1e-3 + 2e-3 |ref| on the head's q|k|v projections and a gate|up pair
at M = 1, 4, 8; empty groups, bf16 outputs and argument errors."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, bf16_round_f64, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


@pytest.mark.parametrize("m", [1, 2, 5, 8])
@pytest.mark.parametrize("ns,k", [((64, 96, 32), 512), ((300, 17, 1000), 2048), ((40,), 4096)])
def test_exact_family_bit_exact(orc, m, ns, k):
    import nvfp4_w4a16_mtp_amd as nv
    parts = [synth.exact_family(200 + 7 * i + m, m, n, k) for i, n in enumerate(ns)]
    x = parts[0][0]                      # one activation block shared by every group
    ws = [_w(c, s, g) for _, c, s, g in parts]
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), ws)
    for (_, c, s, g), y in zip(parts, ys):
        ref = orc.gemv(x, c, s, g)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m", [1, 4, 8])
def test_qkv(orc, m):
    """The head's q (8192 x 2048), k and v (512 x 2048) in one launch."""
    import nvfp4_w4a16_mtp_amd as nv
    shapes = [(8192, 2048), (512, 2048), (512, 2048)]
    ref_parts = []
    for i, (n, k) in enumerate(shapes):
        rng = np.random.default_rng([50 + i, 3])
        ref_parts.append(synth.quantized_domain_weight(rng, n, k))
    x = synth.acts_bf16(60 + m, m, 2048)
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), [_w(*p) for p in ref_parts])
    for (c, s, g), y, nm in zip(ref_parts, ys, "qkv"):
        assert_close(y.cpu().numpy(), orc.gemv(x, c, s, g), f"{nm} m={m}")


@pytest.mark.parametrize("m", [1, 8])
def test_gate_up_pair_matches_single_calls(orc, m):
    """gate|up (1024 x 2048 each): grouped outputs within tolerance of the
    oracle and of the single-weight calls."""
    import nvfp4_w4a16_mtp_amd as nv
    parts = [synth.quantized_domain_weight(np.random.default_rng([70 + i, 3]), 1024, 2048) for i in range(2)]
    x = synth.acts_bf16(80 + m, m, 2048)
    ws = [_w(*p) for p in parts]
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), ws)
    for p, w, y in zip(parts, ws, ys):
        single = nv.w4a16_gemv(dev_bf16(x), w).cpu().numpy()
        ref = orc.gemv(x, *p)
        assert_close(y.cpu().numpy(), ref, "grouped")
        assert_close(single, ref, "single")


def test_empty_groups_and_bf16(orc):
    import nvfp4_w4a16_mtp_amd as nv
    k = 1024
    a = synth.quantized_domain_weight(np.random.default_rng([90, 3]), 130, k)
    b = synth.quantized_domain_weight(np.random.default_rng([91, 3]), 77, k)
    empty = nv.NVFP4Weight.from_parts(torch.zeros((0, k // 2), dtype=torch.uint8, device="cuda"),
                                      torch.zeros((0, k // 16), dtype=torch.uint8, device="cuda"), 1.0)
    x = synth.acts_bf16(92, 3, k)
    ws = [empty, _w(*a), empty, _w(*b), empty]
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), ws, out_dtype=torch.bfloat16)
    assert [tuple(y.shape) for y in ys] == [(3, 0), (3, 130), (3, 0), (3, 77), (3, 0)]
    for p, y in ((a, ys[1]), (b, ys[3])):
        ref = orc.gemv(x, *p)
        ulp = np.abs(bf16_round_f64(ref)) * 2.0 ** -7
        assert (np.abs(y.float().cpu().numpy() - bf16_round_f64(ref)) <= ulp + 1e-30).all()
    # all groups empty: nothing launched, nothing read
    assert [tuple(y.shape) for y in nv.w4a16_gemv_grouped(dev_bf16(x), [empty, empty])] == [(3, 0), (3, 0)]


def test_canaries_around_outputs(orc):
    """No group writes outside its own output."""
    import nvfp4_w4a16_mtp_amd as nv
    k = 512
    parts = [synth.quantized_domain_weight(np.random.default_rng([95 + i, 3]), n, k) for i, n in enumerate((33, 65))]
    x = synth.acts_bf16(97, 2, k)
    buf = torch.full((2 * 33 + 64 + 2 * 65 + 64,), 12345.0, dtype=torch.float32, device="cuda")
    y0 = buf[:66].view(2, 33)
    y1 = buf[66 + 64:66 + 64 + 130].view(2, 65)
    nv.w4a16_gemv_grouped(dev_bf16(x), [_w(*p) for p in parts], outs=[y0, y1])
    host = buf.cpu().numpy()
    assert (host[66:130] == 12345.0).all() and (host[260:] == 12345.0).all()
    assert_close(y0.cpu().numpy(), orc.gemv(x, *parts[0]), "g0")
    assert_close(y1.cpu().numpy(), orc.gemv(x, *parts[1]), "g1")


def test_errors():
    import nvfp4_w4a16_mtp_amd as nv
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    w64 = nv.NVFP4Weight.from_parts(torch.zeros((4, 32), dtype=torch.uint8, device="cuda"),
                                    torch.zeros((4, 4), dtype=torch.uint8, device="cuda"), 1.0)
    w128 = nv.NVFP4Weight.from_parts(torch.zeros((4, 64), dtype=torch.uint8, device="cuda"),
                                     torch.zeros((4, 8), dtype=torch.uint8, device="cuda"), 1.0)
    with pytest.raises(nv.NVFP4Error):
        nv.w4a16_gemv_grouped(x, [])                         # count 0
    with pytest.raises(nv.NVFP4Error):
        nv.w4a16_gemv_grouped(x, [w64] * 9)                  # count > 8
    with pytest.raises(nv.NVFP4Error):
        nv.w4a16_gemv_grouped(x, [w64, w128])                # k differs
    with pytest.raises(nv.NVFP4Error):
        nv.w4a16_gemv_grouped(torch.zeros((9, 64), dtype=torch.bfloat16, device="cuda"), [w64])


@pytest.mark.parametrize("m", [5, 8])
def test_rows_beyond_the_lds_go_in_groups(orc, m):
    """Two weights at K = 17408: round_up(m) rows of activations exceed the
    LDS, so the rows go in groups (5 -> 4 + 1, 8 -> 4 + 4); each group's
    outputs land at its row offset in every output (bit exact on the exact
    family)."""
    import nvfp4_w4a16_mtp_amd as nv
    parts = [synth.exact_family(230 + 5 * i + m, m, n, 17408) for i, n in enumerate((96, 33))]
    x = parts[0][0]
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), [_w(c, s, g) for _, c, s, g in parts])
    for (_, c, s, g), y in zip(parts, ys):
        assert np.array_equal(y.cpu().numpy().view(np.uint32), orc.gemv(x, c, s, g).view(np.uint32))
