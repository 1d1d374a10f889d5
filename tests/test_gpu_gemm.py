"""GPU parity: w4a16_gemm_m128 (C ABI) vs the oracle: bit-exact on the exact-
arithmetic family (bf16 MFMA products are exact), within tolerance on normal
inputs, sampled at the prefill configurations."""
import numpy as np
import pytest
import torch

from tests import synth
from tests.gpu_util import assert_close, bf16_round_f64, dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _w(codes, scales, g_dec):
    import nvfp4_w4a16_mtp_amd as nv
    return nv.NVFP4Weight.from_parts(dev_u8(codes), dev_u8(scales), float(g_dec))


@pytest.mark.parametrize("m,n,k", [(1, 128, 64), (128, 128, 64), (200, 384, 512), (77, 130, 96), (300, 512, 2048),
                                   (512, 128, 64), (600, 200, 96), (1000, 384, 2048),
                                   (300, 32728, 96), (257, 65536, 64)])
def test_exact_family_bit_exact(orc, m, n, k):
    """The last two shapes have 512 or more 256-row tiles: 256-row workgroups."""
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(200 + m, m, n, k)
    y = nv.w4a16_gemm_m128(dev_bf16(x), _w(codes, scales, g)).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m,n,k", [(128, 2048, 4096), (257, 512, 2048), (777, 640, 1024), (513, 22000, 1024)])
def test_random_full(orc, m, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    w = synth.weight_bf16(300 + n, n, k)
    x = synth.acts_bf16(301, m, k)
    codes, scales, glob = orc.quantize(w)
    y = nv.w4a16_gemm_m128(dev_bf16(x), _w(codes, scales, glob[0])).cpu().numpy()
    assert_close(y, orc.gemv(x, codes, scales, glob[0]), f"gemm {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(200, 384, 1024), (64, 640, 4096), (130, 256, 96 * 64)])
def test_split_k_equals_one_pass(orc, m, n, k):
    """Short chunks cut K into slices summed from a workspace; on the exact
    family both that and one pass over K equal the oracle bit for bit."""
    import nvfp4_w4a16_mtp_amd as nv
    assert nv.gemm_workspace(m, n, k, torch.device("cuda")) is not None   # the split path is taken
    x, codes, scales, g = synth.exact_family(210 + m, m, n, k)
    wd = _w(codes, scales, g)
    ys = nv.w4a16_gemm_m128(dev_bf16(x), wd).cpu().numpy()
    y1 = nv.w4a16_gemm_m128(dev_bf16(x), wd, split_k=False).cpu().numpy()
    ref = orc.gemv(x, codes, scales, g)
    assert np.array_equal(ys.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m,n,k,first_tail", [
    (256, 66560, 2048, 65536),     # 520 tall tiles on 512 slots: the last 8 split over K
    (128, 102400, 2048, 98304)])   # 800 tiles on 768 slots: the last 32 split over K
def test_last_round_split_bit_exact(orc, m, n, k, first_tail):
    """With 256 CUs these shapes fill one round of resident workgroups and
    spill a few tiles into a second; with a workspace those tiles split K
    over several workgroups in the same launch (tile-shaped partials, summed
    in slice order).  Exact family: the split call, one pass over K and the
    oracle agree bit for bit -- the oracle on 3000 random outputs and on
    three whole rows of the split tiles, one pass on every output."""
    import nvfp4_w4a16_mtp_amd as nv
    ws = nv.gemm_workspace(m, n, k, torch.device("cuda"))
    assert ws is not None
    x, codes, scales, g = synth.exact_family(220 + m, m, n, k)
    wd = _w(codes, scales, g)
    xd = dev_bf16(x)
    ys = nv.w4a16_gemm_m128(xd, wd, workspace=ws)
    y1 = nv.w4a16_gemm_m128(xd, wd, split_k=False)
    assert torch.equal(ys.view(torch.int32), y1.view(torch.int32))
    rng = np.random.default_rng(221)
    tail_n = np.arange(first_tail, n)
    mi = np.concatenate([rng.integers(0, m, 3000), np.repeat([0, m // 2 + 1, m - 1], tail_n.size)])
    ni = np.concatenate([rng.integers(0, n, 3000), np.tile(tail_n, 3)])
    got = ys[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    ref = orc.gemm_sample(x, codes, scales, g, mi, ni)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_split_k_workspace_too_small():
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(5, 128, 512, 1024)
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        nv.w4a16_gemm_m128(dev_bf16(x), _w(codes, scales, g), workspace=ws)


def test_gemm_m1_equals_gemv(orc):
    import nvfp4_w4a16_mtp_amd as nv
    x, codes, scales, g = synth.exact_family(9, 8, 512, 1024)
    wd = _w(codes, scales, g)
    a = nv.w4a16_gemm_m128(dev_bf16(x), wd).cpu().numpy()
    b = nv.w4a16_gemv(dev_bf16(x), wd).cpu().numpy()
    assert np.array_equal(a, b)


_WEIGHTS = {}


@pytest.mark.parametrize("m", [128, 1024, 8192])
@pytest.mark.parametrize("name,n,k", [("fc", 2048, 4096), ("kv", 512, 2048), ("gate_up", 17408, 5120),
                                      ("down", 5120, 17408)])
def test_prefill_configs_sampled(orc, m, name, n, k):
    import nvfp4_w4a16_mtp_amd as nv
    if name not in _WEIGHTS:
        codes, scales, g = synth.quantized_domain_weight(np.random.default_rng([400, n, k]), n, k)
        _WEIGHTS[name] = (codes, scales, g, _w(codes, scales, g))
    codes, scales, g, wd = _WEIGHTS[name]
    rng = np.random.default_rng(400 + m)
    x = synth.acts_bf16(401 + m, m, k)
    y = nv.w4a16_gemm_m128(dev_bf16(x), wd)
    mi = rng.integers(0, m, 3000)
    ni = rng.integers(0, n, 3000)
    mi[:4] = [0, m - 1, 0, m - 1]
    ni[:4] = [0, n - 1, n - 1, 0]
    got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    ref = orc.gemm_sample(x, codes, scales, g, mi, ni)
    assert_close(got, ref, f"{name} m={m}")


def test_bf16_output(orc):
    import nvfp4_w4a16_mtp_amd as nv
    w = synth.weight_bf16(500, 256, 512)
    x = synth.acts_bf16(501, 130, 512)
    codes, scales, glob = orc.quantize(w)
    wd = _w(codes, scales, glob[0])
    y32 = nv.w4a16_gemm_m128(dev_bf16(x), wd).cpu().numpy()
    yb = nv.w4a16_gemm_m128(dev_bf16(x), wd, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(yb, bf16_round_f64(y32).astype(np.float32))
