"""CPU oracle for the NVFP4 W4A16 MTP draft-head hot path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(the ``nvfp4_w4a16_mtp_amd`` package and its HIP library) never imports it.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, fp64 accumulation);
this module only builds it with gcc and marshals numpy arrays.  Each wrapper
names the page passage its C function follows in that file's comments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: no FMA contraction, no fast-math."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        f32 = ctypes.c_float
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e2m1_decode.argtypes = [ctypes.c_int]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_int]
        L.orc_e2m1_encode.restype = ctypes.c_int
        L.orc_e2m1_encode.argtypes = [f32]
        L.orc_e4m3_encode.restype = ctypes.c_int
        L.orc_e4m3_encode.argtypes = [f32]
        L.orc_bf16_round.restype = f32
        L.orc_bf16_round.argtypes = [f32]
        L.orc_e2m1_encode_array.argtypes = [P, i64, P]
        L.orc_e4m3_encode_array.argtypes = [P, i64, P]
        L.orc_global_scales.argtypes = [P, i64, P]
        L.orc_quantize.argtypes = [P, i64, i64, P, P, P]
        L.orc_dequantize.argtypes = [P, P, f32, i64, i64, P]
        L.orc_gemv.argtypes = [P, i64, P, P, f32, i64, i64, P]
        L.orc_gemm_sample.argtypes = [P, P, P, f32, i64, P, P, i64, P]
        L.orc_lmhead_argmax.argtypes = [P, i64, P, P, f32, i64, i64, ctypes.c_uint32,
                                        P, P, P, P]
        L.orc_lmhead_logprob.argtypes = [P, i64, P, P, f32, i64, i64, ctypes.c_uint32, P]
        L.orc_lmhead_masked.argtypes = [P, i64, P, P, f32, i64, i64, ctypes.c_uint32, P, i64, P, P, P]
        L.orc_embed_rows.argtypes = [P, i64, P, i64, i64, P]
        L.orc_moe_layer.argtypes = [P, i64, P, P, f32, i64, i64, i64, i64,
                                    P, P, P, P, P, P, P, P, P,
                                    P, P, f32, P, P, f32, P, P, f32, i64,
                                    P, P, P, P, P]
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_get_threads.restype = ctypes.c_int
        L.orc_moe.argtypes = [P, i64, P, i64, i64, i64, i64,
                              P, P, P, P, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def set_threads(n: int) -> None:
    """Threads of the loops over independent outputs (results do not depend
    on it)."""
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return lib().orc_get_threads()


# ---- codecs -----------------------------------------------------------------
def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(int(code))


def e4m3_decode(byte: int) -> float:
    return lib().orc_e4m3_decode(int(byte))


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(float(v))


def e4m3_encode(s: float) -> int:
    return lib().orc_e4m3_encode(float(s))


def e2m1_encode_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib().orc_e2m1_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_encode_array(s: np.ndarray) -> np.ndarray:
    s = _c(s, np.float32)
    out = np.zeros(s.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(s), s.size, _p(out))
    return out


def bf16_round(f: float) -> float:
    return lib().orc_bf16_round(float(f))


# ---- quantizer ----------------------------------------------------------------
def global_scales(w_bf16: np.ndarray):
    w = _c(w_bf16, np.uint16)
    out = np.zeros(3, np.float32)
    lib().orc_global_scales(_p(w), w.size, _p(out))
    return out  # g_dec, g_enc, amax


def quantize(w_bf16: np.ndarray):
    """bf16 bits [n, k] -> (codes u8[n, k/2], scales u8[n, k/16], glob f32[3])."""
    w = _c(w_bf16, np.uint16)
    n, k = w.shape
    assert k % 16 == 0
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    glob = np.zeros(3, np.float32)
    lib().orc_quantize(_p(w), n, k, _p(codes), _p(scales), _p(glob))
    return codes, scales, glob


def dequantize(codes, scales, g_dec, n, k):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    out = np.zeros((n, k), np.float64)
    lib().orc_dequantize(_p(codes), _p(scales), float(g_dec), n, k, _p(out))
    return out


# ---- GEMV / GEMM ------------------------------------------------------------------
def gemv(x_bf16, codes, scales, g_dec):
    """x bf16 bits [m, k]; W (codes [n, k/2], scales [n, k/16]) -> fp32 [m, n]."""
    x = _c(x_bf16, np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    m, k = x.shape
    n = codes.shape[0]
    assert codes.shape[1] * 2 == k and scales.shape[1] * 16 == k
    y = np.zeros((m, n), np.float32)
    lib().orc_gemv(_p(x), m, _p(codes), _p(scales), float(g_dec), n, k, _p(y))
    return y


def gemm_sample(x_bf16, codes, scales, g_dec, mi, ni):
    x = _c(x_bf16, np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    k = x.shape[1]
    out = np.zeros(mi.size, np.float32)
    lib().orc_gemm_sample(_p(x), _p(codes), _p(scales), float(g_dec), k, _p(mi), _p(ni),
                          mi.size, _p(out))
    return out


# ---- LM head + argmax ----------------------------------------------------------
def lmhead_argmax(h_bf16, codes, scales, g_dec, vrows=0, flags=0, want_logits=False):
    h = _c(h_bf16, np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    m, k = h.shape
    n = codes.shape[0]
    v = n if vrows <= 0 else min(vrows, n)
    idx = np.zeros(m, np.int32)
    mx = np.zeros(m, np.float32)
    logits = np.zeros((m, v), np.float32) if want_logits else None
    bound = np.zeros((m, v), np.float64) if want_logits else None
    lib().orc_lmhead_argmax(_p(h), m, _p(codes), _p(scales), float(g_dec), k, v, int(flags),
                            _p(idx), _p(mx), _p(logits), _p(bound))
    if want_logits:
        return idx, mx, logits, bound
    return idx, mx


def lmhead_logprob(h_bf16, codes, scales, g_dec, vrows=0, flags=0):
    """Top-1 log-probability per activation row (fp64): the argmax key minus
    the log-sum-exp of all keys of the first `vrows` rows."""
    h = _c(h_bf16, np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    m, k = h.shape
    n = codes.shape[0]
    v = n if vrows <= 0 else min(vrows, n)
    lp = np.zeros(m, np.float64)
    lib().orc_lmhead_logprob(_p(h), m, _p(codes), _p(scales), float(g_dec), k, v, int(flags), _p(lp))
    return lp


def lmhead_masked(h_bf16, codes, scales, g_dec, mask=None, vrows=0, flags=0):
    """Grammar-masked argmax over the first `vrows` rows: mask is uint32
    [m][words] (bit r % 32 of word r / 32 allows row r) or None.  Returns
    (idx, max logit, top-1 log-probability over the allowed rows)."""
    h = _c(h_bf16, np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    m, k = h.shape
    n = codes.shape[0]
    v = n if vrows <= 0 else min(vrows, n)
    words = 0
    if mask is not None:
        mask = _c(mask, np.uint32)
        assert mask.shape[0] == m
        words = mask.shape[1]
    idx = np.zeros(m, np.int32)
    mx = np.zeros(m, np.float32)
    lp = np.zeros(m, np.float64)
    lib().orc_lmhead_masked(_p(h), m, _p(codes), _p(scales), float(g_dec), k, v, int(flags), _p(mask), words,
                            _p(idx), _p(mx), _p(lp))
    return idx, mx, lp


def embed_rows(idx, table_bf16):
    """Rows table[idx[i]] (bf16 bits), zero rows for out-of-range ids."""
    idx = _c(idx, np.int32)
    table = _c(table_bf16, np.uint16)
    vocab, hidden = table.shape
    out = np.zeros((len(idx), hidden), np.uint16)
    lib().orc_embed_rows(_p(idx), len(idx), _p(table), vocab, hidden, _p(out))
    return out


# ---- MoE ------------------------------------------------------------------------------
def moe(x_bf16, router, topk, gate, up, down):
    """gate/up/down: (codes [E, rows, cols/2], scales [E, rows, cols/16], g_dec [E])."""
    x = _c(x_bf16, np.uint16)
    router = _c(router, np.float32)
    m, H = x.shape
    E = router.shape[1]
    gc, gs, gd = (_c(gate[0], np.uint8), _c(gate[1], np.uint8), _c(gate[2], np.float32))
    uc, us, ud = (_c(up[0], np.uint8), _c(up[1], np.uint8), _c(up[2], np.float32))
    dc, ds, dd = (_c(down[0], np.uint8), _c(down[1], np.uint8), _c(down[2], np.float32))
    I = gc.shape[1]
    assert gc.shape == (E, I, H // 2) and dc.shape == (E, H, I // 2)
    y = np.zeros((m, H), np.float32)
    ids = np.zeros((m, topk), np.int32)
    w = np.zeros((m, topk), np.float32)
    lib().orc_moe(_p(x), m, _p(router), E, topk, H, I, _p(gc), _p(gs), _p(gd), _p(uc), _p(us),
                  _p(ud), _p(dc), _p(ds), _p(dd), _p(y), _p(ids), _p(w))
    return y, ids, w


def moe_layer(x_bf16, router, topk, gate, up, down, shared, sgate_bf16=None):
    """The complete MoE layer: router (codes [E, H/2], scales [E, H/16], g_dec)
    -> logits; routed experts gate/up/down as in moe(); shared = (gate, up,
    down), each (codes, scales, g_dec); sgate_bf16: bf16 bits [H] or None.
    Returns (y, ids, wts, logits)."""
    x = _c(x_bf16, np.uint16)
    m, H = x.shape
    rc, rs, rd = _c(router[0], np.uint8), _c(router[1], np.uint8), float(router[2])
    E = rc.shape[0]
    gc, gs, gd = (_c(gate[0], np.uint8), _c(gate[1], np.uint8), _c(gate[2], np.float32))
    uc, us, ud = (_c(up[0], np.uint8), _c(up[1], np.uint8), _c(up[2], np.float32))
    dc, ds, dd = (_c(down[0], np.uint8), _c(down[1], np.uint8), _c(down[2], np.float32))
    I = gc.shape[1]
    (sgc, sgs, sgd), (suc, sus, sud), (sdc, sds, sdd) = shared
    sgc, sgs, suc, sus = (_c(a, np.uint8) for a in (sgc, sgs, suc, sus))
    sdc, sds = _c(sdc, np.uint8), _c(sds, np.uint8)
    Is = sgc.shape[0]
    assert rc.shape == (E, H // 2) and sgc.shape == (Is, H // 2) and sdc.shape == (H, Is // 2)
    sg = None if sgate_bf16 is None else _c(sgate_bf16, np.uint16)
    y = np.zeros((m, H), np.float32)
    ids = np.zeros((m, topk), np.int32)
    wts = np.zeros((m, topk), np.float32)
    logits = np.zeros((m, E), np.float32)
    lib().orc_moe_layer(_p(x), m, _p(rc), _p(rs), rd, E, topk, H, I,
                        _p(gc), _p(gs), _p(gd), _p(uc), _p(us), _p(ud), _p(dc), _p(ds), _p(dd),
                        _p(sgc), _p(sgs), float(sgd), _p(suc), _p(sus), float(sud), _p(sdc), _p(sds), float(sdd), Is,
                        _p(sg), _p(y), _p(ids), _p(wts), _p(logits))
    return y, ids, wts, logits

