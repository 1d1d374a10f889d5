"""GPU parity: moe_w4a16_gemv (C ABI) vs the oracle: top-k ids bit-exact,
routing weights and outputs within |d| <= 1e-3 + 2e-3 |ref|."""
import numpy as np
import pytest

from tests import synth
from tests.gpu_util import assert_close, dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


def _dev_experts(gate, up, down):
    import nvfp4_w4a16_mtp_amd as nv
    import torch

    def glob(g):
        a = np.zeros((len(g), 4), np.float32)
        a[:, 0] = g
        return dev_f32(a)
    return nv.NVFP4Experts(dev_u8(gate[0]), dev_u8(gate[1]), glob(gate[2]), dev_u8(up[0]), dev_u8(up[1]),
                           glob(up[2]), dev_u8(down[0]), dev_u8(down[1]), glob(down[2]))


def _run(orc, experts_np, dev_experts, x, r, topk):
    import nvfp4_w4a16_mtp_amd as nv
    y, ids, w = nv.moe_w4a16_gemv(dev_bf16(x), dev_f32(r), topk, dev_experts)
    ry, rids, rw = orc.moe(x, r, topk, *experts_np)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert_close(w.cpu().numpy(), rw, "routing weights")
    assert_close(y.cpu().numpy(), ry, "moe output")


@pytest.mark.parametrize("m,topk", [(1, 1), (2, 4), (2, 8), (3, 4), (3, 8), (5, 8), (8, 8), (8, 16)])
def test_small(orc, m, topk):
    ex = synth.moe_quantized_experts(1, 32, 256, 128)
    x = synth.acts_bf16(1 + m, m, 256)
    r = synth.router_logits(1 + m, m, 32)
    _run(orc, ex, _dev_experts(*ex), x, r, topk)


def test_ties_in_router(orc):
    ex = synth.moe_quantized_experts(2, 16, 128, 64)
    x = synth.acts_bf16(2, 3, 128)
    r = synth.router_logits(2, 3, 16)
    r[1, [2, 9, 5]] = 4.0
    r[2, :] = 0.5
    _run(orc, ex, _dev_experts(*ex), x, r, 4)


_BIG = {}


@pytest.mark.parametrize("m", [1, 4, 8])
def test_config_256_experts(orc, m):
    """256 experts, hidden 2048, inter 1024, top-8."""
    if "ex" not in _BIG:
        ex = synth.moe_quantized_experts(3, 256, 2048, 1024)
        _BIG["ex"] = (ex, _dev_experts(*ex))
    ex, dex = _BIG["ex"]
    x = synth.acts_bf16(3 + m, m, 2048)
    r = synth.router_logits(3 + m, m, 256)
    _run(orc, ex, dex, x, r, 8)


@pytest.mark.parametrize("m", [3, 4, 8])
def test_several_tiles_per_workgroup_uneven(orc, m):
    """inter 1056: 66 row tiles per (token, slot) pair, more than one round of
    gate/up workgroups holds at these token counts, so a workgroup takes
    several tiles of its pair and the tiles do not divide evenly among them."""
    ex = synth.moe_quantized_experts(5, 64, 512, 1056)
    x = synth.acts_bf16(50 + m, m, 512)
    r = synth.router_logits(50 + m, m, 64)
    _run(orc, ex, _dev_experts(*ex), x, r, 8)
