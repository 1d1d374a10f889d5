"""GPU parity of w4a16_gemv_embed: the GEMV whose activation rows begin with
the embedding rows of the tokens in idx, gathered by its own activation
loads (the next draft step's fc over [embed(draft token) | hidden state],
mtp_head.rs `MtpHead` fields: `embed_from_argmax`; deepseek_v4_mtp.rs
`propose` feeds each draft into the next step).  The oracle computes the
GEMV of the concatenated rows, with its own gather (zero rows for ids
outside the table).  Exact-arithmetic inputs (table and rest rows in
{-3..3}, exact-family weights) are compared bit for bit, on every kernel
the shapes reach: the one-row register path, the LDS path and the K-split
MFMA units (gathered rows never take the persistent grid; the largest
shape is one that would for plain rows); random inputs equal w4a16_gemv of
the concatenated rows bit for bit."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


def _ints(seed, rows, cols):
    rng = np.random.default_rng([seed, 5])
    return synth.f32_to_bf16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("n,k,hidden,vocab", [(2048, 4096, 2048, 3000), (333, 512, 256, 70), (96, 4096, 4096, 50),
                                              (64, 1024, 32, 9), (16387, 2048, 1024, 500)])
def test_exact_family_bit_exact(orc, m, n, k, hidden, vocab):
    import nvfp4_w4a16_mtp_amd as nv
    _, codes, scales, g = synth.exact_family(700 + m, 1, n, k)
    table = _ints(701, vocab, hidden)
    rest = _ints(702 + m, m, k - hidden)
    rng = np.random.default_rng([703, m, n])
    idx = rng.integers(0, vocab, m).astype(np.int32)
    if m >= 3:
        idx[1], idx[2] = -1, vocab          # outside the table: zero rows
    x = np.concatenate([orc.embed_rows(idx, table), rest], axis=1)
    ref = orc.gemv(x, codes, scales, g)
    got = nv.w4a16_gemv_embed(torch.from_numpy(idx).cuda(), dev_bf16(table),
                              dev_bf16(rest) if k > hidden else None, _w(codes, scales, g)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m", [1, 4, 8])
def test_equals_gemv_of_gathered_rows(m):
    """Random bf16 rows, the fc shape: bit-identical to w4a16_gemv over the
    rows embed_from_argmax materializes, in fp32 and bf16 output."""
    import nvfp4_w4a16_mtp_amd as nv
    H = 2048
    w = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(710, 2048, 2 * H)))
    table = dev_bf16(synth.acts_bf16(711, 5000, H))
    rest = dev_bf16(synth.acts_bf16(712 + m, m, H))
    idx = torch.from_numpy(np.random.default_rng(713 + m).integers(0, 5000, m).astype(np.int32)).cuda()
    xin = torch.empty((m, 2 * H), dtype=torch.bfloat16, device="cuda")
    nv.embed_from_argmax(idx, table, out=xin[:, :H])
    xin[:, H:].copy_(rest)
    for dt in (torch.float32, torch.bfloat16):
        a = nv.w4a16_gemv_embed(idx, table, rest, w, out_dtype=dt)
        b = nv.w4a16_gemv(xin, w, out_dtype=dt)
        assert torch.equal(a.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           b.view(torch.int16 if dt == torch.bfloat16 else torch.int32))


def test_errors():
    import nvfp4_w4a16_mtp_amd as nv
    w = nv.nvfp4_quantize(dev_bf16(synth.weight_bf16(720, 64, 512)))
    idx = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        nv.w4a16_gemv_embed(idx, dev_bf16(synth.acts_bf16(721, 10, 256)), dev_bf16(synth.acts_bf16(722, 2, 200)), w)
    with pytest.raises(nv.NVFP4Error, match="hidden"):
        nv.w4a16_gemv_embed(idx, dev_bf16(synth.acts_bf16(723, 10, 40)), dev_bf16(synth.acts_bf16(724, 2, 472)), w)
