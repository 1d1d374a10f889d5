"""A chain of draft steps on the GPU checked against the same chain run by
the oracle.  Each draft feeds the next step (deepseek_v4_mtp.rs, `propose`),
its id staying on the device (mtp_head.rs, `MtpHead` fields:
`embed_from_argmax` and the device id buffer):

    tok_j   = argmax(lm_head h_j)                  (LM head + argmax)
    x_j     = [embed(tok_j) | h_j]                 (embedding gather, bf16)
    h_{j+1} = bf16(fc x_j)                         (W4A16 GEMV, K = 2 H)

The oracle runs the chain with its own argmax, gather and GEMV.  The LM head
gets one planted row per step (codes 7 with the signs of that step's h, the
largest scale), computed on the oracle's chain, so every step's winner is
certified by a margin far above the fp32 bound; the GPU's draft-id log must
equal the oracle's exactly, each gathered row must equal the oracle's gather
bit for bit, and each step's fc output must be within one bf16 ulp of the
oracle's GEMV of the GPU's own input row (plus the fp32 bound).  Three ways
of chaining are checked: argmax then embed_from_argmax, the argmax with the
gather fused into its last workgroup, and the argmax followed by an fc that
gathers the embedding row itself (w4a16_gemv_embed); eagerly and as a HIP
graph of the whole chain."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import bf16_round_f64, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu

H, V, STEPS = 2048, 16384, 6


def _plant_star(codes, scales, h_bits, row):
    hf = synth.bf16_bits_to_f32(h_bits)
    code = (7 | (np.signbit(hf).astype(np.uint8) << 3)).astype(np.uint8)
    codes[row] = (code[0::2] | (code[1::2] << 4)).astype(np.uint8)
    scales[row] = 0x7E


def _oracle_chain(orc, h0, lm, fc, table, plant=False, seed=0):
    """Runs the chain for every activation row of h0 on the oracle.  With
    plant, the LM head rows are overwritten first so that step j of row i
    selects a fresh planted row.  Returns (ids [STEPS][m], h [STEPS + 1])."""
    lm_c, lm_s, lm_g = lm
    rng = np.random.default_rng(seed)
    used = set()
    h = h0.copy()
    ids, hs = [], [h.copy()]
    for j in range(STEPS):
        if plant:
            for i in range(h.shape[0]):
                while True:
                    r = int(rng.integers(0, V))
                    if r not in used:
                        used.add(r)
                        break
                _plant_star(lm_c, lm_s, h[i], r)
        idx, _ = orc.lmhead_argmax(h, lm_c, lm_s, lm_g)
        x = np.concatenate([orc.embed_rows(idx, table), h], axis=1)
        y = orc.gemv(x, *fc)
        h = synth.f32_to_bf16_bits(y)
        ids.append(idx.copy())
        hs.append(h.copy())
    return np.array(ids), hs


def _certify(orc, hs, lm, ids):
    """Every step's winner beats every other row by more than the rigorous
    fp32 bound (so any correct implementation selects it)."""
    gamma = (H + 8) * 2.0 ** -24
    for j in range(STEPS):
        _, _, logits, absb = orc.lmhead_argmax(hs[j], *lm, want_logits=True)
        for i in range(hs[j].shape[0]):
            w = ids[j][i]
            b = gamma * absb[i] + 1e-30
            gap = logits[i, w] - np.delete(logits[i], w)
            assert (gap > b[w] + np.delete(b, w)).all(), (j, i)


def _setup(orc, m):
    rng = np.random.default_rng(90 + m)
    lm_c, lm_s, lm_g = synth.quantized_domain_weight(rng, V, H)
    fc_c, fc_s, fc_g = synth.quantized_domain_weight(rng, H, 2 * H)
    fc = (fc_c, fc_s, np.float32(fc_g * 2))
    table = synth.acts_bf16(91 + m, V, H)
    h0 = synth.acts_bf16(92 + m, m, H)
    lm = (lm_c, lm_s, lm_g)
    ids, hs = _oracle_chain(orc, h0, lm, fc, table, plant=True, seed=93 + m)
    # the chain on the final (fully planted) head, from scratch
    ids2, hs2 = _oracle_chain(orc, h0, lm, fc, table)
    assert np.array_equal(ids, ids2)
    _certify(orc, hs2, lm, ids2)
    return lm, fc, table, h0, ids2


def _fc_within_bound(orc, got_bits, x_bits, fc):
    """The GPU's bf16 output is the rounding of an fp32 sum within the
    rigorous bound (K + 8) 2^-24 * sum |terms| of the exact one: it lies
    within that bound plus one bf16 ulp of the rounded oracle result."""
    _, _, ref, absb = orc.lmhead_argmax(x_bits, *fc, want_logits=True)
    got = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    rb = bf16_round_f64(ref)
    lim = np.abs(rb) * 2.0 ** -7 + (2 * H + 8) * 2.0 ** -24 * absb + 1e-30
    assert (np.abs(got - rb) <= lim).all()


@pytest.mark.parametrize("m", [1, 2])
def test_chain_matches_oracle(orc, m):
    import nvfp4_w4a16_mtp_amd as nv
    lm, fc, table, h0, ref_ids = _setup(orc, m)
    lm_d = nv.NVFP4Weight.from_parts(dev_u8(lm[0]), dev_u8(lm[1]), float(lm[2]))
    fc_d = nv.NVFP4Weight.from_parts(dev_u8(fc[0]), dev_u8(fc[1]), float(fc[2]))
    table_d = dev_bf16(table)
    ws = nv.lmhead_workspace(m, V, "cuda")
    xin = torch.empty((m, 2 * H), dtype=torch.bfloat16, device="cuda")
    hcur = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(m, dtype=torch.int32, device="cuda")
    mx = torch.empty(m, dtype=torch.float32, device="cuda")
    log = torch.zeros((STEPS, m), dtype=torch.int32, device="cuda")
    xlog = torch.empty((STEPS, m, 2 * H), dtype=torch.bfloat16, device="cuda")
    hlog = torch.empty((STEPS, m, H), dtype=torch.bfloat16, device="cuda")
    hprev = torch.empty((STEPS, m, H), dtype=torch.bfloat16, device="cuda")

    h0_d = dev_bf16(h0)

    def chain(mode):
        hcur.copy_(h0_d)
        for j in range(STEPS):
            hprev[j].copy_(hcur)
            if mode == "consumer":
                # the argmax writes the id log; the fc reads the embedding row itself
                nv.lmhead_gemv_argmax(hcur, lm_d, workspace=ws, out_idx=log[j], out_max=mx)
                nv.w4a16_gemv_embed(log[j], table_d, hprev[j], fc_d, out=hcur, out_dtype=torch.bfloat16)
            else:
                if mode == "fused":
                    nv.lmhead_gemv_argmax_embed(hcur, lm_d, table_d, xin[:, :H], id_log=log[j], workspace=ws,
                                                out_idx=idx, out_max=mx)
                else:
                    nv.lmhead_gemv_argmax(hcur, lm_d, workspace=ws, out_idx=idx, out_max=mx)
                    nv.embed_from_argmax(idx, table_d, out=xin[:, :H], id_log=log[j])
                xin[:, H:].copy_(hcur)
                xlog[j].copy_(xin)
                nv.w4a16_gemv(xin, fc_d, out=hcur, out_dtype=torch.bfloat16)
            hlog[j].copy_(hcur)

    def check(mode):
        torch.cuda.synchronize()
        ids = log.cpu().numpy()
        assert np.array_equal(ids, ref_ids), (ids, ref_ids)
        hs = hlog.cpu().view(torch.int16).numpy().view(np.uint16)
        hp = hprev.cpu().view(torch.int16).numpy().view(np.uint16)
        xs = xlog.cpu().view(torch.int16).numpy().view(np.uint16)
        for j in range(STEPS):
            x = np.concatenate([orc.embed_rows(ids[j], table), hp[j]], axis=1)   # the oracle's gather
            if mode != "consumer":
                assert np.array_equal(xs[j], x)                                     # the GPU's, bit for bit
            _fc_within_bound(orc, hs[j], x, fc)                                     # the step's fc GEMV

    for mode in ("separate", "fused", "consumer"):
        log.zero_()
        chain(mode)
        check(mode)
    s = torch.cuda.Stream()
    for mode in ("fused", "consumer"):
        with torch.cuda.stream(s):
            chain(mode)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                chain(mode)
        torch.cuda.synchronize()
        for rep in range(3):
            log.zero_()
            xlog.zero_()
            g.replay()
            check(mode)
            chain("separate")                             # eager work between replays
            check("separate")
