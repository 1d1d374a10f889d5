"""GPU parity: moe_layer_w4a16 (router GEMV + routed experts + sigmoid-gated
shared expert, C ABI) vs the oracle's complete layer.

With a router and activations from the exact-arithmetic family the fp32
router logits are exact on both sides, so the logits and the routing are
compared bit for bit (ties included: the lower expert id first); outputs
and routing weights within |d| <= 1e-3 + 2e-3 |ref|.  On random routers a
token is compared only when its top-k boundary is certified by the fp32
error bound of its logits.  Also: the ungated shared expert, m = 1..8, the
Qwen-shaped expert width (hidden 2048, width 1024)."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _experts(ex):
    import nvfp4_w4a16_mtp_amd as nv

    def glob4(g):
        a = np.zeros((len(g), 4), np.float32)
        a[:, 0] = g
        return torch.from_numpy(a).cuda()
    return nv.NVFP4Experts(*[dev_u8(t) if i % 3 != 2 else glob4(t) for i, t in enumerate([p for proj in ex for p in proj])])


def _shared(rng, H, I):
    return tuple(synth.quantized_domain_weight(rng, r, c) for r, c in ((I, H), (I, H), (H, I)))


@pytest.mark.parametrize("m,topk,E,gated", [(1, 8, 32, True), (4, 8, 32, True), (8, 8, 32, False), (3, 2, 16, True)])
def test_exact_router(orc, m, topk, E, gated):
    import nvfp4_w4a16_mtp_amd as nv
    H, I = 2048, 1024
    x, rc, rs, rg = synth.exact_family(300 + m, m, E, H)
    ex = synth.moe_quantized_experts(301 + m, E, H, I)
    rng = np.random.default_rng([302, m])
    shared = _shared(rng, H, I)
    sgate = synth.acts_bf16(303, 1, H)[0] if gated else None
    y, ids, wts, logits = nv.moe_layer_w4a16(
        dev_bf16(x), _w(rc, rs, rg), topk, _experts(ex), *[_w(*p) for p in shared],
        shared_gate_w=dev_bf16(sgate[None])[0] if gated else None)
    ry, rids, rw, rlogits = orc.moe_layer(x, (rc, rs, rg), topk, *ex, shared, sgate)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), rlogits.view(np.uint32))
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert_close(wts.cpu().numpy(), rw, "weights")
    assert_close(y.cpu().numpy(), ry, f"layer m={m}")


@pytest.mark.parametrize("m", [1, 8])
def test_random_router_certified(orc, m):
    import nvfp4_w4a16_mtp_amd as nv
    H, I, E, topk = 2048, 1024, 64, 8
    rng = np.random.default_rng([310, m])
    rc, rs, rg = synth.quantized_domain_weight(rng, E, H)
    rg = np.float32(rg * 3000.0)                          # logits of order one
    x = synth.acts_bf16(311 + m, m, H)
    ex = synth.moe_quantized_experts(312, E, H, I)
    shared = _shared(rng, H, I)
    sgate = synth.acts_bf16(313, 1, H)[0]
    y, ids, wts, logits = nv.moe_layer_w4a16(dev_bf16(x), _w(rc, rs, rg), topk, _experts(ex),
                                             *[_w(*p) for p in shared], shared_gate_w=dev_bf16(sgate[None])[0])
    ry, rids, rw, rlogits = orc.moe_layer(x, (rc, rs, rg), topk, *ex, shared, sgate)
    assert_close(logits.cpu().numpy(), rlogits, "router logits")
    # fp32 bound of a logit: (K + 8) 2^-24 * g * sum |x w|
    _, _, _, absb = orc.lmhead_argmax(x, rc, rs, rg, want_logits=True)
    bound = (H + 8) * 2.0 ** -24 * absb
    ids, y = ids.cpu().numpy(), y.cpu().numpy()
    checked = 0
    for t in range(m):
        srt = np.argsort(-rlogits[t], kind="stable")
        kth, nxt = srt[topk - 1], srt[topk]
        if rlogits[t, kth] - rlogits[t, nxt] > bound[t, kth] + bound[t, nxt]:
            assert np.array_equal(ids[t], rids[t])
            assert_close(y[t], ry[t], f"token {t}")
            checked += 1
    assert checked >= max(1, m // 2)


def test_errors():
    import nvfp4_w4a16_mtp_amd as nv
    H, I, E = 256, 128, 8
    ex = synth.moe_quantized_experts(320, E, H, I)
    rng = np.random.default_rng(321)
    shared = _shared(rng, H, I)
    x = dev_bf16(synth.acts_bf16(322, 1, H))
    router = _w(*synth.quantized_domain_weight(rng, E + 1, H))      # wrong expert count
    with pytest.raises(nv.NVFP4Error):
        nv.moe_layer_w4a16(x, router, 2, _experts(ex), *[_w(*p) for p in shared])
    router = _w(*synth.quantized_domain_weight(rng, E, H))
    bad = _shared(rng, H, I + 32)                                   # shared width differs
    with pytest.raises(nv.NVFP4Error):
        nv.moe_layer_w4a16(x, router, 2, _experts(ex), *[_w(*p) for p in bad])
