"""Seeded synthetic inputs for the NVFP4 W4A16 MTP hot path.

This module only draws random numbers and lays them out; it performs none of
the method's arithmetic (no quantization, no dot products, no argmax).  The
tests feed the same arrays to the CPU oracle and to the HIP library.

Recipe (stated once here, used everywhere):
* ``numpy.random.default_rng(seed)``; draws happen in the order W, x, router
  logits, plant positions.
* Normal draws are fp32 ``standard_normal`` times the stated deviation, then
  rounded to bf16 (nearest-even) -- bf16 weights ~N(0, 0.02), activations
  ~N(0, 1), router logits fp32 ~N(0, 1).
* Weights "in the quantized domain" (used where a test needs hundreds of
  expert matrices without running a quantizer on the CPU) draw E2M1 codes
  from a fixed histogram close to that of quantized normal blocks, E4M3
  scales from a narrow band of bytes and a power-of-two-free global scale.
* The exact-arithmetic family draws x from {-3..3}, power-of-two block scales
  in [2^-2, 2^2] and a power-of-two global scale, so that every partial sum
  of every dot product is exactly representable in fp32.
* The scale-range family keeps x and the codes of the exact family but draws
  the block scale bytes of a row from one E4M3 binade (8 consecutive bytes)
  that depends on the row; over the rows the binades cover every byte
  0x00-0x7E (zero and subnormal scales included), half the rows with the sign
  bit set.  Within one binade the scales share one quantum, so sums stay
  exact.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).ravel()
    out = np.empty(u.shape, np.uint16)
    step = 1 << 24
    for lo in range(0, u.size, step):
        v = u[lo:lo + step]
        out[lo:lo + step] = ((v + (((v >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def weight_bf16(seed: int, n: int, k: int, std: float = 0.02) -> np.ndarray:
    """bf16 weight [n, k] ~ N(0, std)."""
    return normal_bf16(np.random.default_rng(seed), (n, k), std)


def acts_bf16(seed: int, m: int, k: int, std: float = 1.0) -> np.ndarray:
    """bf16 activations [m, k] ~ N(0, std); the stream is offset from the
    weight stream of the same seed."""
    return normal_bf16(np.random.default_rng([seed, 1]), (m, k), std)


def router_logits(seed: int, m: int, e: int) -> np.ndarray:
    return np.random.default_rng([seed, 2]).standard_normal((m, e), dtype=np.float32)


# E2M1 magnitude codes 0..7 drawn with probabilities close to what
# quantizing a normal block with its max mapped to 6 gives, as counts out of
# 128 (one random byte per element: low 7 bits pick the magnitude through
# this table, the top bit is the sign).
_CODE_COUNTS = [14, 24, 22, 19, 19, 14, 11, 5]
_MAG_LUT = np.repeat(np.arange(8, dtype=np.uint8), _CODE_COUNTS)
assert _MAG_LUT.size == 128
_CODE_LUT = (_MAG_LUT[np.arange(256) & 0x7F] | ((np.arange(256) >> 7) << 3)).astype(np.uint8)
# one random uint16 -> one packed byte (two codes, low byte -> even k)
_PAIR_LUT = (_CODE_LUT[np.arange(65536) & 0xFF] | (_CODE_LUT[np.arange(65536) >> 8] << 4)).astype(np.uint8)


def quantized_domain_weight(rng: np.random.Generator, n: int, k: int):
    """Synthetic NVFP4 weight drawn directly as codes/scales/global.
    Returns (codes u8[n, k/2], scales u8[n, k/16], g_dec f32)."""
    codes = _PAIR_LUT[rng.integers(0, 65536, size=(n, k // 2), dtype=np.uint16)]
    # E4M3 bytes 0x50..0x7E: scales roughly 8 .. 448, the band quantized
    # normal weights land in with a global scale of amax/2688.
    scales = rng.integers(0x50, 0x7F, size=(n, k // 16), dtype=np.uint8)
    g_dec = np.float32(rng.uniform(1e-5, 3e-5))
    return codes, scales, g_dec


def moe_quantized_experts(seed: int, num_experts: int, hidden: int, inter: int):
    """Stacked synthetic NVFP4 experts: gate/up [E, inter, hidden], down
    [E, hidden, inter].  Each returned as (codes, scales, g_dec[E])."""
    rng = np.random.default_rng([seed, 3])
    out = []
    for rows, cols in ((inter, hidden), (inter, hidden), (hidden, inter)):
        c = _PAIR_LUT[rng.integers(0, 65536, size=(num_experts, rows, cols // 2), dtype=np.uint16)]
        s = rng.integers(0x50, 0x7F, size=(num_experts, rows, cols // 16), dtype=np.uint8)
        g = rng.uniform(1e-5, 3e-5, size=num_experts).astype(np.float32)
        out.append((c, s, g))
    return out


def exact_family(seed: int, m: int, n: int, k: int):
    """Inputs whose dot products are exact in fp32 in any summation order:
    x in {-3..3}, codes uniform over all 16, block scales 2^-2..2^2 (E4M3
    bytes 0x28, 0x30, 0x38, 0x40, 0x48), g_dec a power of two.
    Returns (x bf16 bits [m, k], codes, scales, g_dec)."""
    rng = np.random.default_rng([seed, 4])
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = (rng.integers(5, 10, size=(n, k // 16)) << 3).astype(np.uint8)
    g_dec = np.float32(2.0 ** int(rng.integers(-6, 1)))
    x = f32_to_bf16_bits(rng.integers(-3, 4, size=(m, k)).astype(np.float32))
    return x, codes, scales, g_dec




# Scale windows: the E4M3 bytes of one binade, [8 j, 8 j + 7] (byte 0x7F
# excluded), j = (r + seed) mod 16 for row r, so 16 consecutive rows cover
# every byte 0x00..0x7E.  The values of window j are multiples of one
# quantum q_j (2^-9 for j <= 1, else 2^(j - 10)) and at most 15 q_j, so a
# dot product with x in {-3..3} and any E2M1 codes has every partial sum a
# multiple of q_j / 2 below 288 * 15 * (K / 16) * q_j: under 2^24 quanta for
# K up to 17408, exact in fp32 in any summation order.
def scale_window_bytes(rng: np.random.Generator, n: int, nblocks: int, seed: int = 0,
                       signed: bool = True, binades=None) -> np.ndarray:
    """binades: the windows j to cycle through (default all 16)."""
    js = np.arange(16) if binades is None else np.asarray(list(binades), np.int64)
    w0 = 8 * js[(np.arange(n, dtype=np.int64) + seed) % len(js)]
    b = np.minimum(w0[:, None] + rng.integers(0, 8, size=(n, nblocks)), 0x7E).astype(np.uint8)
    if signed:
        b |= (rng.integers(0, 2, size=(n, 1)) << 7).astype(np.uint8)
    return b


def scale_range_family(seed: int, m: int, n: int, k: int, signed: bool = True, binades=None):
    """The exact family with block scales over the whole E4M3 range: x in
    {-3..3}, codes uniform over all 16, scale bytes from per-row windows (see
    scale_window_bytes; zero, subnormal and normal scales, negative ones when
    `signed`), g_dec a power of two.  Every dot product is exact in fp32 in
    any summation order.  Returns (x bf16 bits [m, k], codes, scales, g_dec)."""
    rng = np.random.default_rng([seed, 7])
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = scale_window_bytes(rng, n, k // 16, seed, signed, binades)
    g_dec = np.float32(2.0 ** int(rng.integers(-4, 3)))
    x = f32_to_bf16_bits(rng.integers(-3, 4, size=(m, k)).astype(np.float32))
    return x, codes, scales, g_dec


def scale_decode_rows(m: int, k: int, seed: int = 0):
    """One weight row per E4M3 scale byte (0x00..0x7E, then 0x80..0xFE: 254
    rows), every code 1.0 (E2M1 0x2), and activation rows that are one-hot
    in every 16-element block (value +-1 or +-2 at a random position).  Output
    (row r, activation i) = g_dec * e4m3(byte r) * sum of x[i] in closed form.
    Returns (x bf16 bits [m, k], codes, scales, bytes [254])."""
    rng = np.random.default_rng([seed, 8])
    byt = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    n = byt.size
    codes = np.full((n, k // 2), 0x22, np.uint8)
    scales = np.repeat(byt[:, None], k // 16, axis=1)
    xf = np.zeros((m, k), np.float32)
    for i in range(m):
        pos = rng.integers(0, 16, size=k // 16) + 16 * np.arange(k // 16)
        xf[i, pos] = rng.choice(np.array([-2.0, -1.0, 1.0, 2.0], np.float32), size=k // 16)
    return f32_to_bf16_bits(xf), codes, scales, byt


def moe_scale_window_experts(seed: int, num_experts: int, hidden: int, inter: int):
    """Stacked synthetic experts like moe_quantized_experts, but expert e
    draws all its block-scale bytes from the window [8 (e % 16), 8 (e % 16) + 7]
    (byte 0x7F excluded), so the experts together cover every scale byte,
    zero and subnormal ones included.  Its g_dec is the power of two that puts
    its largest weight magnitude (6 times the window's top scale) near 0.03,
    so every expert contributes at the same magnitude."""
    rng = np.random.default_rng([seed, 9])
    out = []
    w0 = 8 * (np.arange(num_experts) % 16)
    top = np.minimum(w0 + 7, 0x7E)
    e, mt = (top >> 3) & 15, top & 7
    vmax = np.where(e == 0, mt * 2.0 ** -9, (1 + mt / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    g = (2.0 ** np.round(np.log2(0.03 / (6.0 * vmax)))).astype(np.float32)
    for rows, cols in ((inter, hidden), (inter, hidden), (hidden, inter)):
        c = _PAIR_LUT[rng.integers(0, 65536, size=(num_experts, rows, cols // 2), dtype=np.uint16)]
        s = (w0[:, None, None] + rng.integers(0, 8, size=(num_experts, rows, cols // 16))).astype(np.int64)
        s = np.minimum(s, 0x7E).astype(np.uint8)
        out.append((c, s, g.copy()))
    return out


def plant_lmhead_rows(codes: np.ndarray, scales: np.ndarray, h_bf16: np.ndarray, seed: int,
                      n_near: int = 4, dup: bool = False, scale_byte: int = 0x7E,
                      vrows: int | None = None) -> dict:
    """Overwrite LM-head rows in place so that every token has a known winner.

    For token i a row ``star`` gets E2M1 code 7 (magnitude 6) with the sign of
    h[i, k] at every k and the E4M3 byte ``scale_byte`` in every block.
    ``n_near`` copies of it have one code stepped down to 6 (magnitude 4) at
    the k's with the largest |h[i, k]|.  With ``dup`` two exact copies go one
    below and one above ``star``.  Rows are only placed inside [0, vrows).
    """
    n, half = codes.shape
    k = half * 2
    v = n if vrows is None else min(vrows, n)
    m = h_bf16.shape[0]
    rng = np.random.default_rng([seed, 6])
    hf = bf16_bits_to_f32(h_bf16)
    used: set[int] = set()

    def fresh(lo: int, hi: int) -> int:
        while True:
            r = int(rng.integers(lo, hi))
            if r not in used:
                used.add(r)
                return r

    info = {"star": [], "near": [], "near_k": [], "dups": [], "scale_byte": scale_byte}
    for i in range(m):
        sign = (np.signbit(hf[i]).astype(np.uint8) << 3)
        code = (7 | sign).astype(np.uint8)
        row_codes = (code[0::2] | (code[1::2] << 4)).astype(np.uint8)
        star = fresh(v // 4, (3 * v) // 4)
        codes[star] = row_codes
        scales[star] = scale_byte
        order = np.argsort(-np.abs(hf[i]), kind="stable")[:n_near]
        near, near_k = [], []
        for kk in order:
            r = fresh(0, v)
            c2 = code.copy()
            c2[kk] = 6 | sign[kk]
            codes[r] = (c2[0::2] | (c2[1::2] << 4)).astype(np.uint8)
            scales[r] = scale_byte
            near.append(r)
            near_k.append(int(kk))
        dups = []
        if dup:
            for lo, hi in ((0, star), (star + 1, v)):
                r = fresh(lo, hi)
                codes[r] = row_codes
                scales[r] = scale_byte
                dups.append(r)
        info["star"].append(star)
        info["near"].append(near)
        info["near_k"].append(near_k)
        info["dups"].append(dups)
    assert k == h_bf16.shape[1]
    return info
