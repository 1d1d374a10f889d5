"""GPU parity for device-resident draft chaining: the grammar-masked LM-head
argmax (lmhead_gemv_argmax_masked) against the oracle's masked scan, the
embedding gather (embed_from_argmax) against the oracle's gather, and a chain
of draft steps captured in one HIP graph (argmax -> embedding -> next step's
GEMV, the draft ids recorded on the device) against the same steps run one by
one with a host readback after each, on every replay."""
import math

import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _mask_bits(allowed):
    m, v = allowed.shape
    words = np.zeros((m, (v + 31) // 32), np.uint32)
    for i in range(m):
        r = np.flatnonzero(allowed[i])
        np.bitwise_or.at(words[i], r // 32, (np.uint32(1) << (r % 32).astype(np.uint32)))
    return words


def _dev_mask(words):
    return torch.from_numpy(words.view(np.int32)).cuda()


def _certified(orc, h, codes, scales, g, allowed, idx, ridx):
    """idx must equal ridx unless the best allowed logits are within the fp32
    error bound of each other; then idx must be allowed and within the bound."""
    _, _, logits, absb = orc.lmhead_argmax(h, codes, scales, g, want_logits=True)
    gamma = (h.shape[1] + 8) * 2.0 ** -24
    for i in range(h.shape[0]):
        if not allowed[i].any():
            assert idx[i] == 0
            continue
        a = np.flatnonzero(allowed[i])
        bound = gamma * absb[i] + 1e-30
        top = logits[i, ridx[i]]
        close = a[(top - logits[i, a] <= bound[ridx[i]] + bound[a]) & (a != ridx[i])]
        if len(close) == 0:
            assert idx[i] == ridx[i], (i, idx[i], ridx[i])
        else:
            assert allowed[i, idx[i]] and logits[i, idx[i]] >= top - 2 * bound.max()


@pytest.mark.parametrize("m,v,k,density,bf16", [(1, 3000, 512, 0.3, False), (4, 5000, 2048, 0.01, False),
                                                 (8, 2049, 1024, 0.5, True), (3, 700, 512, 1.0, False)])
def test_masked_random(orc, m, v, k, density, bf16):
    import nvfp4_w4a16_mtp_amd as nv
    rng = np.random.default_rng([m, v, k])
    codes, scales, g = synth.quantized_domain_weight(rng, v, k)
    g = np.float32(g * 400.0)
    h = synth.acts_bf16(5 + m, m, k)
    allowed = rng.random((m, v)) < density
    if m >= 3:
        allowed[1, :] = False                     # nothing allowed: the pad index 0
        allowed[2, :] = False
        allowed[2, v - 1] = True                  # exactly one token, the last row
    words = _mask_bits(allowed)
    idx, mx, lp = nv.lmhead_gemv_argmax_masked(dev_bf16(h), _w(codes, scales, g), _dev_mask(words), bf16_keys=bf16,
                                               with_logprob=True)
    idx, mx, lp = idx.cpu().numpy(), mx.cpu().numpy(), lp.cpu().numpy()
    ridx, rmx, rlp = orc.lmhead_masked(h, codes, scales, g, mask=words, flags=int(bf16))
    _certified(orc, h, codes, scales, g, allowed, idx, ridx)
    for i in range(m):
        if not allowed[i].any():
            assert idx[i] == 0 and np.isnan(lp[i]) and np.isnan(rlp[i])
        elif idx[i] == ridx[i]:
            assert_close(mx[i:i + 1], rmx[i:i + 1], "max")
            assert_close(lp[i:i + 1], rlp[i:i + 1], "logprob")
    if m >= 3:
        assert idx[2] == v - 1 and lp[2] == 0.0


def test_all_allowed_equals_unmasked(orc):
    import nvfp4_w4a16_mtp_amd as nv
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(3), 4000, 2048)
    h = synth.acts_bf16(4, 5, 2048)
    wd = _w(codes, scales, g)
    words = np.full((5, (4000 + 31) // 32), 0xFFFFFFFF, np.uint32)
    i0, m0 = nv.lmhead_gemv_argmax(dev_bf16(h), wd)
    i1, m1 = nv.lmhead_gemv_argmax_masked(dev_bf16(h), wd, _dev_mask(words))
    assert np.array_equal(i0.cpu().numpy(), i1.cpu().numpy())
    assert np.array_equal(m0.cpu().numpy().view(np.uint32), m1.cpu().numpy().view(np.uint32))


def test_full_head_grammar_mask(orc):
    """151936 x 2048 head, 1% of the vocabulary allowed plus the planted
    winner, which must be found; a short mask (first 1000 words) too."""
    import nvfp4_w4a16_mtp_amd as nv
    v, k = 151936, 2048
    codes, scales, g = synth.quantized_domain_weight(np.random.default_rng(50), v, k)
    h = synth.acts_bf16(51, 2, k)
    info = synth.plant_lmhead_rows(codes, scales, h, seed=52, n_near=4)
    rng = np.random.default_rng(53)
    allowed = rng.random((2, v)) < 0.01
    allowed[0, info["star"][0]] = True
    allowed[1, info["star"][1]] = False           # row 1: the planted winner is not allowed
    words = _mask_bits(allowed)
    idx, mx = nv.lmhead_gemv_argmax_masked(dev_bf16(h), _w(codes, scales, g), _dev_mask(words))
    idx = idx.cpu().numpy()
    ridx, rmx, _ = orc.lmhead_masked(h, codes, scales, g, mask=words)
    assert idx[0] == info["star"][0] == ridx[0]
    _certified(orc, h, codes, scales, g, allowed, idx, ridx)
    short = np.ascontiguousarray(words[:, :1000])
    idx, _ = nv.lmhead_gemv_argmax_masked(dev_bf16(h), _w(codes, scales, g), _dev_mask(short))
    ridx, _, _ = orc.lmhead_masked(h, codes, scales, g, mask=short)
    al = np.zeros_like(allowed)
    al[:, :32000] = allowed[:, :32000]
    _certified(orc, h, codes, scales, g, al, idx.cpu().numpy(), ridx)


def test_embed_from_argmax(orc):
    import nvfp4_w4a16_mtp_amd as nv
    rng = np.random.default_rng(60)
    vocab, hidden = 5000, 2048
    table = rng.integers(0, 65536, size=(vocab, hidden), dtype=np.uint16)
    ids = np.array([0, 4999, 17, -3, 5000, 17], np.int32)
    m = len(ids)
    buf = torch.full((m, 2 * hidden + 64), 7, dtype=torch.int16, device="cuda")   # canaries around the rows
    out = buf.view(torch.bfloat16)[:, 32:32 + hidden]
    log = torch.full((m,), -99, dtype=torch.int32, device="cuda")
    nv.embed_from_argmax(torch.from_numpy(ids).cuda(), dev_bf16(table), out=out, id_log=log)
    host = buf.cpu().numpy().view(np.uint16)
    assert np.array_equal(host[:, 32:32 + hidden], orc.embed_rows(ids, table))
    assert (host[:, :32] == 7).all() and (host[:, 32 + hidden:] == 7).all()
    assert np.array_equal(log.cpu().numpy(), ids)


def test_chain_in_a_graph():
    """Four chained draft steps in one HIP graph: h_{j+1} = bf16(fc([embed(tok_j) | h_j])),
    tok_{j+1} = argmax(lm_head h_{j+1}); ids recorded on the device.  Every
    replay equals the same steps run eagerly with a readback after each."""
    import nvfp4_w4a16_mtp_amd as nv
    H, V, steps = 2048, 32768, 4
    rng = np.random.default_rng(70)
    lm = _w(*synth.quantized_domain_weight(rng, V, H))
    fc_c, fc_s, fc_g = synth.quantized_domain_weight(rng, H, 2 * H)
    fc = _w(fc_c, fc_s, np.float32(fc_g * 40))
    table = dev_bf16(synth.acts_bf16(71, V, H))
    h0 = dev_bf16(synth.acts_bf16(72, 1, H))
    ws = nv.lmhead_workspace(1, V, "cuda")

    xin = torch.empty((1, 2 * H), dtype=torch.bfloat16, device="cuda")   # [embed | hidden] input of fc
    hcur = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    mx = torch.empty(1, dtype=torch.float32, device="cuda")
    log = torch.zeros(steps, dtype=torch.int32, device="cuda")

    def chain(readback=None):
        hcur.copy_(h0)
        for j in range(steps):
            nv.lmhead_gemv_argmax(hcur, lm, workspace=ws, out_idx=idx, out_max=mx)
            if readback is not None:
                readback.append(int(idx.item()))
            nv.embed_from_argmax(idx, table, out=xin[:, :H], id_log=log[j:j + 1])
            xin[:, H:].copy_(hcur)
            nv.w4a16_gemv(xin, fc, out=hcur, out_dtype=torch.bfloat16)

    eager = []
    chain(eager)
    torch.cuda.synchronize()
    assert log.cpu().numpy().tolist() == eager
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        chain()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            chain()
    torch.cuda.synchronize()
    for rep in range(3):
        log.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert log.cpu().numpy().tolist() == eager, rep
        again = []
        chain(again)                                # eager work between replays
        torch.cuda.synchronize()
        assert again == eager


@pytest.mark.parametrize("m,masked,logprob,hidden,table_rows", [
    (1, False, False, 1024, 7000), (3, True, True, 1024, 7000), (8, False, True, 1024, 7000),
    (8, False, False, 7168, 7000),     # 14 units a lane per row: several load batches
    (5, True, False, 1000, 3000),      # 125 units a row (not a multiple of 64); ids past the table
    (1, False, False, 8, 7000)])       # one 16-byte unit a row
def test_argmax_embed_fused(orc, m, masked, logprob, hidden, table_rows):
    """lmhead_gemv_argmax_embed equals lmhead_gemv_argmax(_masked/_logprob)
    followed by embed_from_argmax, bit for bit, gathers what the oracle
    gathers (a zero row for an id past the table), and writes nothing else."""
    import nvfp4_w4a16_mtp_amd as nv
    v, k = 6000, 2048
    rng = np.random.default_rng([80, m])
    codes, scales, g = synth.quantized_domain_weight(rng, v, k)
    wd = _w(codes, scales, np.float32(g * 300))
    h = dev_bf16(synth.acts_bf16(81 + m, m, k))
    table_h = synth.acts_bf16(82, table_rows, hidden)
    table = dev_bf16(table_h)
    mask = _dev_mask(_mask_bits(rng.random((m, v)) < 0.2)) if masked else None
    if masked:
        ri, rm, rlp = nv.lmhead_gemv_argmax_masked(h, wd, mask, with_logprob=True)
    else:
        ri, rm, rlp = nv.lmhead_gemv_argmax_logprob(h, wd)
    ref_rows = nv.embed_from_argmax(ri, table)
    buf = torch.full((m, hidden + 64), 5, dtype=torch.int16, device="cuda")
    out = buf.view(torch.bfloat16)[:, 16:16 + hidden]
    log = torch.full((m,), -1, dtype=torch.int32, device="cuda")
    lp = torch.empty(m, dtype=torch.float32, device="cuda") if logprob else None
    idx, mx = nv.lmhead_gemv_argmax_embed(h, wd, table, out, allow_mask=mask, id_log=log, out_logprob=lp)
    assert np.array_equal(idx.cpu().numpy(), ri.cpu().numpy())
    assert np.array_equal(mx.cpu().numpy().view(np.uint32), rm.cpu().numpy().view(np.uint32))
    if logprob:
        assert np.array_equal(lp.cpu().numpy().view(np.uint32), rlp.cpu().numpy().view(np.uint32))
    host = buf.cpu().numpy()
    assert np.array_equal(host[:, 16:16 + hidden].view(np.uint16), ref_rows.cpu().view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(host[:, 16:16 + hidden].view(np.uint16), orc.embed_rows(ri.cpu().numpy(), table_h))
    assert (host[:, :16] == 5).all() and (host[:, 16 + hidden:] == 5).all()
    assert np.array_equal(log.cpu().numpy(), ri.cpu().numpy())


def test_fused_chain_in_a_graph():
    """The chain of test_chain_in_a_graph with the gather fused into the LM
    head gives the same draft ids on every replay."""
    import nvfp4_w4a16_mtp_amd as nv
    H, V, steps = 2048, 32768, 4
    rng = np.random.default_rng(70)
    lm = _w(*synth.quantized_domain_weight(rng, V, H))
    fc_c, fc_s, fc_g = synth.quantized_domain_weight(rng, H, 2 * H)
    fc = _w(fc_c, fc_s, np.float32(fc_g * 40))
    table = dev_bf16(synth.acts_bf16(71, V, H))
    h0 = dev_bf16(synth.acts_bf16(72, 1, H))
    ws = nv.lmhead_workspace(1, V, "cuda")
    xin = torch.empty((1, 2 * H), dtype=torch.bfloat16, device="cuda")
    hcur = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    mx = torch.empty(1, dtype=torch.float32, device="cuda")
    log = torch.zeros(steps, dtype=torch.int32, device="cuda")

    def unfused(readback):
        hcur.copy_(h0)
        for j in range(steps):
            nv.lmhead_gemv_argmax(hcur, lm, workspace=ws, out_idx=idx, out_max=mx)
            readback.append(int(idx.item()))
            nv.embed_from_argmax(idx, table, out=xin[:, :H])
            xin[:, H:].copy_(hcur)
            nv.w4a16_gemv(xin, fc, out=hcur)

    def fused():
        hcur.copy_(h0)
        for j in range(steps):
            nv.lmhead_gemv_argmax_embed(hcur, lm, table, xin[:, :H], id_log=log[j:j + 1], workspace=ws, out_idx=idx,
                                        out_max=mx)
            xin[:, H:].copy_(hcur)
            nv.w4a16_gemv(xin, fc, out=hcur)

    eager = []
    unfused(eager)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fused()
        torch.cuda.synchronize()
        assert log.cpu().numpy().tolist() == eager
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fused()
    torch.cuda.synchronize()
    for rep in range(3):
        log.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert log.cpu().numpy().tolist() == eager, rep
        again = []
        unfused(again)
        torch.cuda.synchronize()
        assert again == eager
