"""Pins for the oracle's complete MoE layer (router GEMV + routed experts +
sigmoid-gated shared expert), CPU only.

Pins: an independent numpy implementation of the whole layer on a small
shape (weights dequantized from the OCP code tables, fp64 arithmetic, bf16
rounding of the expert activations by torch); the logits equal the pinned
GEMV and, with a zero shared expert, the output equals the pinned routed
MoE bit for bit; the gate at sigmoid = 1 and 1/2 in closed form.
"""
import numpy as np
import pytest
import torch

from tests import synth

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _deq(codes, scales, g):
    c = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    c[:, 0::2], c[:, 1::2] = codes & 15, codes >> 4
    return E2M1[c & 7] * np.where(c & 8, -1.0, 1.0) * np.repeat(E4M3[scales], 16, axis=1) * float(g)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()


def _layer(E=8, H=64, I=32, Is=64, m=3, seed=0):
    rng = np.random.default_rng(seed)
    router = synth.quantized_domain_weight(rng, E, H)
    router = (router[0], router[1], np.float32(router[2] * 2000))   # logits of order 1
    ex = synth.moe_quantized_experts(seed + 1, E, H, I)
    shared = tuple(synth.quantized_domain_weight(rng, r, c) for r, c in ((Is, H), (Is, H), (H, Is)))
    x = synth.acts_bf16(seed + 2, m, H)
    return router, ex, shared, x


def _numpy_layer(x, router, topk, ex, shared, sgate):
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    logits = (xf @ _deq(*router).T).astype(np.float32)
    (gc, gs, gd), (uc, us, ud), (dc, ds, dd) = ex
    E = gc.shape[0]
    y = np.zeros((x.shape[0], x.shape[1]))
    for t in range(x.shape[0]):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:topk]
        sel = np.array([logits[t, e] for e in order], np.float64)
        w = np.exp(sel - sel[0]) / np.exp(sel - sel[0]).sum()
        acc = np.zeros(x.shape[1])
        for j, e in enumerate(order):
            g = (xf[t] @ _deq(gc[e], gs[e], gd[e]).T).astype(np.float32).astype(np.float64)
            u = (xf[t] @ _deq(uc[e], us[e], ud[e]).T).astype(np.float32).astype(np.float64)
            a = _bf16(g / (1 + np.exp(-g)) * u)
            d = (a @ _deq(dc[e], ds[e], dd[e]).T).astype(np.float32)
            acc += np.float32(w[j]) * d.astype(np.float64)
        y[t] = acc.astype(np.float32)
        (sgc, sgs, sgd), (suc, sus, sud), (sdc, sds, sdd) = shared
        g = (xf[t] @ _deq(sgc, sgs, sgd).T).astype(np.float32).astype(np.float64)
        u = (xf[t] @ _deq(suc, sus, sud).T).astype(np.float32).astype(np.float64)
        a = _bf16(g / (1 + np.exp(-g)) * u)
        d = (a @ _deq(sdc, sds, sdd).T).astype(np.float32).astype(np.float64)
        s = 1.0 if sgate is None else 1.0 / (1.0 + np.exp(-(synth.bf16_bits_to_f32(sgate).astype(np.float64) @ xf[t])))
        y[t] = y[t] + s * d
    return y, logits


@pytest.mark.parametrize("topk,gated", [(1, False), (2, True), (4, True)])
def test_independent_numpy(orc, topk, gated):
    router, ex, shared, x = _layer(seed=topk)
    sgate = synth.acts_bf16(9, 1, x.shape[1])[0] if gated else None
    y, ids, wts, logits = orc.moe_layer(x, router, topk, *ex, shared, sgate)
    ry, rlogits = _numpy_layer(x, router, topk, ex, shared, sgate)
    assert np.allclose(logits, rlogits, rtol=1e-6, atol=1e-7)
    assert np.allclose(y, ry, rtol=1e-5, atol=1e-6)


def test_logits_and_routed_part_match_pinned_functions(orc):
    router, ex, shared, x = _layer(seed=5)
    zero_down = (np.zeros_like(shared[2][0]), shared[2][1], shared[2][2])
    y, ids, wts, logits = orc.moe_layer(x, router, 3, *ex, (shared[0], shared[1], zero_down))
    assert np.array_equal(logits.view(np.uint32), orc.gemv(x, *router).view(np.uint32))
    ry, rids, rw = orc.moe(x, logits, 3, *ex)
    assert np.array_equal(ids, rids) and np.array_equal(wts, rw)
    assert np.array_equal(y.view(np.uint32), ry.view(np.uint32))


def test_gate_closed_forms(orc):
    router, ex, shared, x = _layer(seed=7)
    H = x.shape[1]
    y1, *_ = orc.moe_layer(x, router, 2, *ex, shared, None)
    # a gate whose logit is huge (positive inputs, gate 64): sigmoid == 1 exactly in fp64
    xpos = synth.f32_to_bf16_bits(np.abs(synth.bf16_bits_to_f32(x)) + 0.5)
    yb, *_ = orc.moe_layer(xpos, router, 2, *ex, shared, synth.f32_to_bf16_bits(np.full(H, 64.0, np.float32)))
    yu, *_ = orc.moe_layer(xpos, router, 2, *ex, shared, None)
    assert np.array_equal(yb, yu)
    # a zero gate: sigmoid(0) = 1/2
    zero_down = (np.zeros_like(shared[2][0]), shared[2][1], shared[2][2])
    yr, *_ = orc.moe_layer(x, router, 2, *ex, (shared[0], shared[1], zero_down))
    yh, *_ = orc.moe_layer(x, router, 2, *ex, shared, np.zeros(H, np.uint16))
    assert np.allclose(yh - yr, 0.5 * (y1 - yr), rtol=1e-5, atol=1e-6)
