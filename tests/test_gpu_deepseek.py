"""GPU parity on DeepSeek-shaped heads (hidden 7168, vocabulary 129280,
256-expert MoE with expert width 2048): the LM-head GEMV + argmax (and its
log-probability), the routed MoE and the decode GEMV, against the oracle.
K = 7168 is not a multiple of 2048, so these take the generic K loop of the
GEMV core; m = 8 needs more than 64 KiB of LDS for the activation image."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu

H, V, I = 7168, 129280, 2048


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


@pytest.mark.parametrize("m", [1, 4, 8])
def test_gemv(orc, m):
    import nvfp4_w4a16_mtp_amd as nv
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng([110, m]), 1536, H)
    x = synth.acts_bf16(111 + m, m, H)
    y = nv.w4a16_gemv(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    assert_close(y, orc.gemv(x, codes, scales, g), f"gemv 1536x{H} m={m}")


@pytest.mark.parametrize("m", [1, 8])
def test_lmhead_reduced_rows(orc, m):
    """The first 8192 rows of a 129280 x 7168 head: planted winners, log-probability."""
    import nvfp4_w4a16_mtp_amd as nv
    vr = 8192
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(120), vr, H)
    g = np.float32(g * 200.0)
    h = synth.acts_bf16(121, m, H)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=122, n_near=4)
    idx, mx, lp = nv.lmhead_gemv_argmax_logprob(dev_bf16(h), _w(codes, scales, g))
    assert list(idx.cpu().numpy()) == [info["star"][i] for i in range(m)]
    ridx, rmx = orc.lmhead_argmax(h, codes, scales, g)
    assert_close(mx.cpu().numpy(), rmx, "max logit")
    assert_close(lp.cpu().numpy(), orc.lmhead_logprob(h, codes, scales, g), "logprob")


def test_lmhead_full_vocabulary(orc):
    """All 129280 rows at m = 1 with a planted winner near the end."""
    import nvfp4_w4a16_mtp_amd as nv
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(130), V, H)
    h = synth.acts_bf16(131, 1, H)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=132, n_near=4)
    idx, mx = nv.lmhead_gemv_argmax(dev_bf16(h), _w(codes, scales, g))
    assert int(idx.item()) == info["star"][0]
    _, rmx = orc.lmhead_argmax(h, codes, scales, g)
    assert_close(mx.cpu().numpy(), rmx, "max logit")


@pytest.mark.parametrize("m,topk", [(1, 8), (4, 8), (8, 8)])
def test_moe(orc, m, topk):
    """32 experts of the DeepSeek expert shape (gate/up 2048 x 7168, down
    7168 x 2048); m = 8 stages 8 activation rows of 7168 in LDS."""
    import nvfp4_w4a16_mtp_amd as nv
    E = 32
    ex = synth.moe_quantized_experts(140 + m, E, H, I)
    x = synth.acts_bf16(141 + m, m, H)
    r = synth.router_logits(142 + m, m, E)

    def glob4(g):
        a = np.zeros((len(g), 4), np.float32)
        a[:, 0] = g
        return torch.from_numpy(a).cuda()
    dex = nv.NVFP4Experts(*[dev_u8(t) if i % 3 != 2 else glob4(t) for i, t in enumerate([p for proj in ex for p in proj])])
    y, ids, wts = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), topk, dex)
    ry, rids, rw = orc.moe(x, r, topk, *ex)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert_close(wts.cpu().numpy(), rw, "weights")
    assert_close(y.cpu().numpy(), ry, f"moe m={m}")


def _routed_union(r, topk):
    """Experts in some token's top-k (ascending): restricted to them, every
    token keeps its own top-k, in the same order (random logits, no ties)."""
    return np.unique(np.argsort(-r, axis=1, kind="stable")[:, :topk])


@pytest.mark.parametrize("m", [1, 4, 8])
def test_moe_256_experts_full_width(orc, m):
    """All 256 experts of 2048 x 7168 / 7168 x 2048 on the device (the
    benchmarked stack, 6.3 GB of NVFP4): the experts some token routes to
    hold synthetic weights, the others zeros (a kernel that read one would
    change the result).  The oracle runs on the routed experts with the
    router logits restricted to them; its ids map back through the
    ascending expert list.  256 experts give each routing lane four."""
    import nvfp4_w4a16_mtp_amd as nv
    E = 256
    x = synth.acts_bf16(150 + m, m, H)
    r = synth.router_logits(151 + m, m, E)
    sel = _routed_union(r, 8)
    rng = np.random.default_rng([152, m])
    parts = []
    for rows, cols in ((I, H), (I, H), (H, I)):
        codes = torch.zeros((E, rows, cols // 2), dtype=torch.uint8, device="cuda")
        scales = torch.zeros((E, rows, cols // 16), dtype=torch.uint8, device="cuda")
        glob = torch.zeros((E, 4), dtype=torch.float32, device="cuda")
        cs, ss, gs = [], [], []
        for e in sel:
            c, s, g = synth.quantized_domain_weight(rng, rows, cols)
            codes[int(e)] = dev_u8(c)
            scales[int(e)] = dev_u8(s)
            glob[int(e), 0] = float(g)
            cs.append(c)
            ss.append(s)
            gs.append(g)
        parts.append((codes, scales, glob))
        parts.append((np.stack(cs), np.stack(ss), np.array(gs, np.float32)))
    dex = nv.NVFP4Experts(*parts[0], *parts[2], *parts[4])
    y, ids, wts = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), 8, dex)
    ry, rids, rw = orc.moe(x, np.ascontiguousarray(r[:, sel]), 8, parts[1], parts[3], parts[5])
    assert np.array_equal(ids.cpu().numpy(), sel[rids])
    assert_close(wts.cpu().numpy(), rw, "weights")
    assert_close(y.cpu().numpy(), ry, f"moe 256 experts m={m}")


@pytest.mark.parametrize("m", [4, 8])
def test_lmhead_full_vocabulary_rows(orc, m):
    """All 129280 rows at m = 4 (dot2 units) and 8 (MFMA units: K = 7168 is
    a whole number of 1024-wide load rounds) with planted winners and
    duplicates below them; the maximum logit within tolerance."""
    import nvfp4_w4a16_mtp_amd as nv
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng([160, m]), V, H)
    h = synth.acts_bf16(161 + m, m, H)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=162 + m, n_near=4, dup=True)
    idx, mx = nv.lmhead_gemv_argmax(dev_bf16(h), _w(codes, scales, g))
    idx = idx.cpu().numpy()
    for i in range(m):
        assert idx[i] == min([info["star"][i]] + info["dups"][i])
    ridx, rmx = orc.lmhead_argmax(h, codes, scales, g)
    assert np.array_equal(idx, ridx)
    assert_close(mx.cpu().numpy(), rmx, "max logit")
