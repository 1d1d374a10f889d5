"""Pins for the oracle's MoE expert GEMV with top-k routing (CPU only).

new.rs (`MtpHead::new`) names the generic MoE path as top-k softmax routing,
a SiLU-gated product and a weighted sum, with NVFP4 expert gate/up
[inter, hidden] and down [hidden, inter] matrices.  Pins: brute-force top-k
with planted ties, softmax normalisation, identical experts, top-1 = the
plain SwiGLU FFN computed with numpy, and permutation invariance.
"""
import numpy as np
import pytest
import torch

from tests import synth

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

E, H, I = 16, 128, 64


def _experts(seed):
    return synth.moe_quantized_experts(seed, E, H, I)


def _dense(codes, scales, g):
    n = codes.shape[0]
    c = np.empty((n, codes.shape[1] * 2), np.int64)
    c[:, 0::2], c[:, 1::2] = codes & 15, codes >> 4
    return E2M1[c & 7] * np.where(c & 8, -1.0, 1.0) * np.repeat(E4M3[scales], 16, axis=1) * float(g)


def test_topk_bruteforce_and_ties(orc):
    gate, up, down = _experts(1)
    x = synth.acts_bf16(1, 3, H)
    r = synth.router_logits(1, 3, E)
    r[1, [2, 9, 5]] = 4.0           # planted three-way tie at the top: order 2, 5, 9
    r[2, :] = 0.5                   # all equal: ids 0..k-1
    y, ids, w = orc.moe(x, r, 4, gate, up, down)
    for t in range(3):
        ref = np.lexsort((np.arange(E), -r[t].astype(np.float64)))[:4]
        assert list(ids[t]) == list(ref)
    assert list(ids[1][:3]) == [2, 5, 9] and list(ids[2]) == [0, 1, 2, 3]
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    sel = np.take_along_axis(r, ids, axis=1).astype(np.float64)
    ref_w = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref_w /= ref_w.sum(axis=1, keepdims=True)
    assert np.allclose(w, ref_w, rtol=1e-6, atol=1e-7)


def _swiglu_numpy(xrow, gd, ud, dd):
    xf = synth.bf16_bits_to_f32(xrow).astype(np.float64)
    g = (gd @ xf).astype(np.float32).astype(np.float64)
    u = (ud @ xf).astype(np.float32).astype(np.float64)
    a = torch.from_numpy((g / (1 + np.exp(-g)) * u).astype(np.float32)).to(torch.bfloat16).double().numpy()
    return dd @ a


def test_top1_is_plain_swiglu(orc):
    gate, up, down = _experts(2)
    x = synth.acts_bf16(2, 2, H)
    r = synth.router_logits(2, 2, E)
    y, ids, w = orc.moe(x, r, 1, gate, up, down)
    assert np.array_equal(w, np.ones((2, 1), np.float32))
    for t in range(2):
        e = ids[t, 0]
        ref = _swiglu_numpy(x[t], _dense(gate[0][e], gate[1][e], gate[2][e]),
                            _dense(up[0][e], up[1][e], up[2][e]),
                            _dense(down[0][e], down[1][e], down[2][e]))
        assert np.allclose(y[t], ref, rtol=2e-3, atol=1e-4)


def test_identical_experts(orc):
    gate, up, down = _experts(3)
    same = [tuple(np.broadcast_to(p[..., :1, :, :] if p.ndim == 3 else p[:1], p.shape).copy()
                  for p in proj) for proj in (gate, up, down)]
    x = synth.acts_bf16(3, 2, H)
    r = synth.router_logits(3, 2, E)
    y8, _, _ = orc.moe(x, r, 8, *same)
    y1, _, _ = orc.moe(x, r, 1, *same)
    assert np.allclose(y8, y1, rtol=1e-6, atol=1e-7)


def test_permutation_invariance(orc):
    gate, up, down = _experts(4)
    x = synth.acts_bf16(4, 4, H)
    r = synth.router_logits(4, 4, E)
    perm = np.random.default_rng(4).permutation(E)
    pg = tuple(p[perm] for p in gate)
    pu = tuple(p[perm] for p in up)
    pd = tuple(p[perm] for p in down)
    y, ids, w = orc.moe(x, r, 8, gate, up, down)
    yp, idsp, wp = orc.moe(x, r[:, perm], 8, pg, pu, pd)
    assert np.array_equal(y, yp) and np.array_equal(w, wp)
    assert np.array_equal(perm[idsp], ids)
