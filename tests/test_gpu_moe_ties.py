"""GPU parity of the MoE routing under ties: equal router logits inside the
range of experts one lane holds (with E > 64 a lane sorts several experts'
logits, so the lowest-id rule inside a lane rests on that sort), across
lanes, at the top-k boundary, all-equal rows and +0 / -0 (equal under
IEEE comparison).  The selection rule is the oracle's: top-k by fp32 logit,
descending, the lower expert id first among equal logits (the scan order of
`moe_topk_softmax` named in new.rs, `MtpHead::new`).  topk_ids are compared
bit for bit; weights and outputs within |d| <= 1e-3 + 2e-3 |ref|.  One token
takes the one-launch path, where the ids come from the down workgroups'
routing; more tokens the two-launch path, where workgroup (0, 0) of the
gate/up pass publishes them (and every gate/up workgroup selects its own
token's experts up to its slot)."""
import math

import numpy as np
import pytest

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


def _dev_experts(gate, up, down):
    import nvfp4_w4a16_mtp_amd as nv

    def glob(g):
        a = np.zeros((len(g), 4), np.float32)
        a[:, 0] = g
        return dev_f32(a)
    return nv.NVFP4Experts(dev_u8(gate[0]), dev_u8(gate[1]), glob(gate[2]), dev_u8(up[0]), dev_u8(up[1]),
                           glob(up[2]), dev_u8(down[0]), dev_u8(down[1]), glob(down[2]))


def _tied_router(seed, m, e):
    """Per token (cycling over four patterns) router logits with ties; `per`
    is the number of experts one of 64 lanes holds (ceil(E / 64))."""
    per = math.ceil(e / 64)
    last = e - 1
    r = synth.router_logits(seed, m, e)
    for t in range(m):
        kind = t % 4
        if kind == 0:
            # one lane's experts all equal and six more across lanes: 6 + per
            # tied candidates for 8 places -> the lowest ids among them win
            r[t, 5 * per:6 * per] = 6.0
            r[t, [1, 17 * per + 1, 33 * per, 40 * per + per - 1, 63 * per % e, last]] = 6.0
        elif kind == 1:
            # ties across lanes only, exactly at ranks 6..9 (the boundary)
            r[t, [3, 90 % e, 150 % e, 201 % e, 4 * per + 1]] = np.array([8.0, 7.9, 7.8, 7.7, 7.6], np.float32)
            r[t, [2 * per, 30 * per + per - 1, 50 * per, last]] = 7.5
        elif kind == 2:
            # every logit equal, half of them -0: experts 0 .. k-1
            r[t, :] = 0.0
            r[t, 1::2] = -0.0
        else:
            # equal logits inside one lane at the boundary, the rest distinct
            r[t, [7, 8 * per + 2, 100 % e, 230 % e, 9]] = np.array([9.0, 8.9, 8.8, 8.7, 8.6], np.float32)
            r[t, 12 * per:12 * per + per] = 8.0
            r[t, 12 * per - 1] = 8.0
    return r


@pytest.mark.parametrize("e", [256, 600])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8])
def test_ties(orc, e, m):
    import nvfp4_w4a16_mtp_amd as nv
    ex = synth.moe_quantized_experts(11, e, 256, 128)
    dex = _dev_experts(*ex)
    x = synth.acts_bf16(12 + m, m, 256)
    r = _tied_router(13 + m, m, e)
    for topk in (8, 3):
        y, ids, w = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), topk, dex)
        ry, rids, rw = orc.moe(x, r, topk, *ex)
        assert np.array_equal(ids.cpu().numpy(), rids), (topk, ids.cpu().numpy(), rids)
        assert_close(w.cpu().numpy(), rw, "routing weights")
        assert_close(y.cpu().numpy(), ry, "moe output")
    # the all-equal token selects experts 0 .. k-1 in order
    if m >= 3:
        assert rids[2].tolist() == list(range(3))


def test_ties_config_shape(orc):
    """The configuration's experts (256 of 1024 x 2048), one token and eight,
    with the tie patterns."""
    import nvfp4_w4a16_mtp_amd as nv
    ex = synth.moe_quantized_experts(14, 256, 2048, 1024)
    dex = _dev_experts(*ex)
    for m in (1, 8):
        x = synth.acts_bf16(15 + m, m, 2048)
        r = _tied_router(16 + m, m, 256)
        y, ids, w = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), 8, dex)
        ry, rids, rw = orc.moe(x, r, 8, *ex)
        assert np.array_equal(ids.cpu().numpy(), rids)
        assert_close(y.cpu().numpy(), ry, "moe output")
