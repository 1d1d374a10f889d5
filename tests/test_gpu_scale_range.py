"""GPU parity over the whole E4M3 block-scale range, in every kernel that
decodes block scales: the GEMV (one-row register path, LDS path, generic and
K-split loops, wide workgroups, persistent grid with dot2 and MFMA units,
rows in groups), the grouped GEMV, the LM head (dot2 and MFMA units, both key
modes, log-probability, grammar mask), the prefill GEMM (128- and 256-row
tiles, K split) and the MoE (gate/up and down).

The quantizer applies `quantize_bf16_to_nvfp4` to every projection, router
and expert matrix of the head (new.rs, `MtpHead::new`), and for rows much
smaller than the tensor maximum it emits zero and subnormal E4M3 scales, so
every consumer must decode bytes 0x00-0x7E.  The scale-range family draws
each row's scales from one E4M3 binade, the binades of the rows covering
every byte; its dot products are exact in fp32, so fp32 outputs and argmax
results are compared bit for bit.  One-hot activations give a closed form
per scale byte.  GPU-quantized heavy-tailed weights (the quantizer's own
subnormal scales) are checked element by element against the rigorous fp32
accumulation bound."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _e4m3_torch(byt):
    """E4M3FN decode by torch's float8 type (independent of both sides)."""
    t = torch.from_numpy(np.ascontiguousarray(byt, np.uint8)).view(torch.float8_e4m3fn)
    return t.float().numpy().astype(np.float64)


# ---------------------------------------------------------------- decode table
@pytest.mark.parametrize("m,k", [(1, 2048), (1, 96), (2, 512), (4, 1024), (8, 2048), (3, 5120)])
def test_decode_table_gemv(orc, m, k):
    """One row per scale byte (254 of them), codes 1.0, one-hot activations:
    y[i][r] = g_dec * e4m3(byte r) * sum_k x[i][k], exactly."""
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, byt = synth.scale_decode_rows(m, k, seed=m + k)
    g = np.float32(0.25)
    y = nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(_bits(y), _bits(ref))
    xs = synth.bf16_bits_to_f32(x).astype(np.float64).sum(axis=1)
    closed = (0.25 * xs[:, None] * _e4m3_torch(byt)[None, :]).astype(np.float32)
    assert np.array_equal(y, closed)          # values (a zero scale gives +0 or -0)


@pytest.mark.parametrize("m", [1, 2, 5, 8])
def test_decode_table_gemm_and_grouped(orc, m):
    """The same table through the prefill GEMM and the grouped GEMV."""
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, byt = synth.scale_decode_rows(m, 1024, seed=40 + m)
    g = np.float32(2.0)
    wd = _w(codes, scales, g)
    ref = orc.gemv(x, codes, scales, g)
    y = nv.w4a16_gemm_m128(dev_bf16(x), wd).cpu().numpy()
    assert np.array_equal(_bits(y), _bits(ref))
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), [wd, wd])
    for yy in ys:
        assert np.array_equal(_bits(yy.cpu().numpy()), _bits(ref))


# ---------------------------------------------------------------- GEMV paths
GEMV_SHAPES = [
    (1, 2050, 2048),     # one row, activations in registers, fixed chunk count, K split over wavefronts
    (1, 333, 96),        # one row, generic loop
    (2, 333, 512), (3, 96, 4096), (5, 700, 1024), (8, 333, 512),   # LDS image, fixed and generic
    (1, 333, 5120), (2, 200, 7168), (4, 90, 3072),                  # K split, pipelined loop
    (2, 700, 17408), (4, 333, 17408), (8, 120, 5120),               # wide workgroups
    (1, 16387, 2048), (2, 49155, 256), (4, 8195, 1024), (8, 8195, 2048), (6, 20000, 2048),  # persistent grid
    (8, 301, 17408),                                                # rows in two groups
]


@pytest.mark.parametrize("m,n,k", GEMV_SHAPES)
def test_gemv_bit_exact(orc, m, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.scale_range_family(300 + m, m, n, k)
    wd = _w(codes, scales, g)
    y = nv.w4a16_gemv(dev_bf16(x), wd).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(_bits(y), _bits(ref))
    yb = nv.w4a16_gemv(dev_bf16(x), wd, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(yb, torch.from_numpy(ref).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("m", [1, 4, 8])
def test_grouped_bit_exact(orc, m):
    import nvfp4_w4a16_mtp_amd as nv
    parts = [synth.scale_range_family(320 + 3 * i + m, m, n, 2048) for i, n in enumerate((1000, 160, 160))]
    x = parts[0][0]
    ys = nv.w4a16_gemv_grouped(dev_bf16(x), [_w(c, s, g) for _, c, s, g in parts])
    for (_, c, s, g), y in zip(parts, ys):
        assert np.array_equal(_bits(y.cpu().numpy()), _bits(orc.gemv(x, c, s, g)))


# ---------------------------------------------------------------- LM head
LM_SHAPES = [(1, 20000, 2048), (1, 7000, 512), (2, 9000, 2048), (3, 5000, 1024), (4, 3000, 512),
             (8, 12000, 2048), (8, 700, 9216)]


@pytest.mark.parametrize("binades", [None, (0, 1)])
@pytest.mark.parametrize("m,v,k", LM_SHAPES)
def test_lmhead_bit_exact(orc, m, v, k, binades):
    """Exact logits: index and maximum bit-exact in both key modes.  With
    binades (0, 1) every row has zero, subnormal or smallest-normal scales,
    so the decode of those bytes alone decides the winner."""
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.scale_range_family(340 + m + v, m, v, k, binades=binades)
    wd = _w(codes, scales, g)
    for bf16 in (False, True):
        idx, mx = nv.lmhead_gemv_argmax(dev_bf16(x), wd, bf16_keys=bf16)
        ridx, rmx = orc.lmhead_argmax(x, codes, scales, g, flags=int(bf16))
        assert np.array_equal(idx.cpu().numpy(), ridx), bf16
        assert np.array_equal(_bits(mx.cpu().numpy()), _bits(rmx)), bf16


@pytest.mark.parametrize("m,v,k", [(1, 20000, 2048), (4, 5000, 1024), (8, 6000, 2048)])
def test_lmhead_logprob_and_mask(orc, m, v, k):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, _ = synth.scale_range_family(360 + m, m, v, k, binades=(0, 1, 2))
    g = np.float32(0.5)                    # logits of a few units: the log-sum-exp sees many rows
    wd = _w(codes, scales, g)
    idx, mx, lp = nv.lmhead_gemv_argmax_logprob(dev_bf16(x), wd)
    ridx, rmx = orc.lmhead_argmax(x, codes, scales, g)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(_bits(mx.cpu().numpy()), _bits(rmx))
    assert_close(lp.cpu().numpy(), orc.lmhead_logprob(x, codes, scales, g), "log-probability")
    rng = np.random.default_rng(361 + m)
    allowed = rng.random((m, v)) < 0.3
    words = np.zeros((m, (v + 31) // 32), np.uint32)
    for i in range(m):
        r = np.flatnonzero(allowed[i])
        np.bitwise_or.at(words[i], r // 32, (np.uint32(1) << (r % 32).astype(np.uint32)))
    dm = torch.from_numpy(words.view(np.int32)).cuda()
    idx, mx, lp = nv.lmhead_gemv_argmax_masked(dev_bf16(x), wd, dm, with_logprob=True)
    ridx, rmx, rlp = orc.lmhead_masked(x, codes, scales, g, mask=words)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(_bits(mx.cpu().numpy()), _bits(rmx))
    assert_close(lp.cpu().numpy(), rlp, "masked log-probability")


# ---------------------------------------------------------------- GEMM
@pytest.mark.parametrize("m,n,k", [(1, 128, 64), (128, 254, 2048), (200, 384, 512), (1000, 384, 2048),
                                   (300, 32728, 96), (257, 65536, 64), (130, 1024, 17408)])
def test_gemm_bit_exact(orc, m, n, k):
    """The last three: 256-row tiles (more than 512 tiles) and a K split."""
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.scale_range_family(380 + m, m, n, k)
    y = nv.w4a16_gemm_m128(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    assert np.array_equal(_bits(y), _bits(orc.gemv(x, codes, scales, g)))


@pytest.mark.parametrize("m,n,k", [(200, 384, 1024), (64, 640, 4096)])
def test_gemm_split_k_bit_exact(orc, m, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    assert nv.gemm_workspace(m, n, k, torch.device("cuda")) is not None
    x, codes, scales, g = synth.scale_range_family(390 + m, m, n, k)
    wd = _w(codes, scales, g)
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(_bits(nv.w4a16_gemm_m128(dev_bf16(x), wd).cpu().numpy()), _bits(ref))
    assert np.array_equal(_bits(nv.w4a16_gemm_m128(dev_bf16(x), wd, split_k=False).cpu().numpy()), _bits(ref))


# ---------------------------------------------------------------- MoE
def _dev_experts(gate, up, down):
    import nvfp4_w4a16_mtp_amd as nv

    def glob(g):
        a = np.zeros((len(g), 4), np.float32)
        a[:, 0] = g
        return dev_f32(a)
    return nv.NVFP4Experts(dev_u8(gate[0]), dev_u8(gate[1]), glob(gate[2]), dev_u8(up[0]), dev_u8(up[1]),
                           glob(up[2]), dev_u8(down[0]), dev_u8(down[1]), glob(down[2]))


def _planted_router(seed, m, e):
    """Router logits whose top-8 of token t are experts of the binades
    8 t .. 8 t + 7 (mod 16): token 0 routes to the zero/subnormal and small
    binades, token 1 to the large ones, and so on."""
    r = synth.router_logits(seed, m, e)
    for t in range(m):
        for j in range(8):
            ex = 16 * ((3 * t + 5 * j) % (e // 16)) + (8 * t + j) % 16
            r[t, ex] = 5.0 + 0.25 * j
    return r


_BIG = {}


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_moe_config_scale_windows(orc, m):
    """256 experts of 1024 x 2048 / 2048 x 1024, top-8; expert e's scales all
    lie in binade e % 16 and its global scale evens out the magnitudes."""
    import nvfp4_w4a16_mtp_amd as nv
    if "ex" not in _BIG:
        ex = synth.moe_scale_window_experts(5, 256, 2048, 1024)
        _BIG["ex"] = (ex, _dev_experts(*ex))
    ex, dex = _BIG["ex"]
    x = synth.acts_bf16(400 + m, m, 2048)
    r = _planted_router(401 + m, m, 256)
    y, ids, w = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), 8, dex)
    ry, rids, rw = orc.moe(x, r, 8, *ex)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert set((rids % 16).ravel().tolist()) >= set(range(min(16, 8 * m)))
    assert_close(w.cpu().numpy(), rw, "routing weights")
    assert_close(y.cpu().numpy(), ry, "moe output")


@pytest.mark.parametrize("m,topk", [(1, 8), (3, 4), (8, 8)])
def test_moe_small_scale_windows(orc, m, topk):
    import nvfp4_w4a16_mtp_amd as nv
    ex = synth.moe_scale_window_experts(6, 32, 256, 128)
    x = synth.acts_bf16(410 + m, m, 256)
    r = synth.router_logits(411 + m, m, 32)
    y, ids, w = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), topk, _dev_experts(*ex))
    ry, rids, rw = orc.moe(x, r, topk, *ex)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert_close(y.cpu().numpy(), ry, "moe output")


# ------------------------------------------- quantizer output into consumers
def _heavy_tailed(seed, n, k):
    """bf16 weights whose rows span five decades: the quantizer gives the
    small rows zero and subnormal block scales."""
    f = synth.bf16_bits_to_f32(synth.weight_bf16(seed, n, k))
    f = f * np.float32(10.0) ** np.random.default_rng(seed).uniform(-5.5, 0, (n, 1)).astype(np.float32)
    return synth.f32_to_bf16_bits(f)


def _within_bound(got, ref, absb, k):
    """|got - ref| <= (K + 8) 2^-24 * g_dec * sum |terms|: the rigorous fp32
    accumulation bound of each output, whatever its magnitude."""
    lim = (k + 8) * 2.0 ** -24 * absb + 1e-38
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert (err <= lim).all(), (err / lim).max()


@pytest.mark.parametrize("m", [1, 4, 8])
def test_quantized_subnormal_scales_through_consumers(orc, m):
    import nvfp4_w4a16_mtp_amd as nv
    n, k = 4096, 2048
    w = _heavy_tailed(420, n, k)
    q = nv.nvfp4_quantize(dev_bf16(w))
    codes, scales, glob = orc.quantize(w)
    assert np.array_equal(q.scales.cpu().numpy(), scales) and np.array_equal(q.codes.cpu().numpy(), codes)
    assert (scales == 0).any() and ((scales > 0) & (scales < 8)).any()   # zero and subnormal scales occur
    x = synth.acts_bf16(421 + m, m, k)
    _, _, logits, absb = orc.lmhead_argmax(x, codes, scales, glob[0], want_logits=True)
    _within_bound(nv.w4a16_gemv(dev_bf16(x), q).cpu().numpy(), logits, absb, k)
    _within_bound(nv.w4a16_gemm_m128(dev_bf16(x), q).cpu().numpy(), logits, absb, k)
    # the LM head over the small-scale rows only (the rows below 1e-3 of the max)
    small = np.flatnonzero(np.abs(synth.bf16_bits_to_f32(w)).max(axis=1) < 1e-3 * np.abs(synth.bf16_bits_to_f32(w)).max())
    assert small.size > 100
    sc, ss = np.ascontiguousarray(codes[small]), np.ascontiguousarray(scales[small])
    ws = nv.NVFP4Weight(dev_u8(sc), dev_u8(ss), q.glob, small.size, k)
    idx, mx = nv.lmhead_gemv_argmax(dev_bf16(x), ws)
    ridx, rmx, lg, ab = orc.lmhead_argmax(x, sc, ss, glob[0], want_logits=True)
    gamma = (k + 8) * 2.0 ** -24
    for i in range(m):
        b = gamma * ab[i] + 1e-38
        top = lg[i, ridx[i]]
        gap = top - np.delete(lg[i], ridx[i])
        if (gap > b[ridx[i]] + np.delete(b, ridx[i])).all():
            assert idx.cpu().numpy()[i] == ridx[i]
        else:
            assert lg[i, idx.cpu().numpy()[i]] >= top - 2 * b.max()
