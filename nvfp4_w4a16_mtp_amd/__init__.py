"""NVFP4 W4A16 MTP draft-head hot path on AMD gfx950 (MI355X).

Thin ctypes binding over ``libnvfp4_mtp.so`` (C ABI in include/nvfp4_mtp.h).
It only marshals arguments: every step of every operation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  If the
library is not built the calls raise -- there is no fallback.

Operations (same names as the C ABI):
  nvfp4_quantize               bf16 W[n, k] -> NVFP4Weight (codes, scales, global)
  w4a16_gemv                   x[m<=8, k] @ W^T
  w4a16_gemv_grouped           the GEMV for several weights sharing x (q|k|v, gate|up)
  w4a16_gemv_embed             the GEMV over [embedding rows of device ids | x_rest]
  w4a16_gemm_m128              x[m, k] @ W^T for prompt-sized m (bf16 MFMA)
  lmhead_gemv_argmax           argmax over the first V rows of h @ W^T
  lmhead_gemv_argmax_logprob   ... plus the top-1 log-probability
  lmhead_gemv_argmax_masked    ... restricted to a grammar's allowed tokens
  lmhead_gemv_argmax_embed     ... with the draft tokens' embedding rows gathered
  lmhead_gemv_argmax_noalloc   lmhead_gemv_argmax on the library's own static scratch
  lmhead_gemv_argmax_fc        ... then the next draft step's fc over the chosen token's embedding row
  embed_from_argmax            embedding rows of device-resident token ids
  moe_w4a16_gemv               top-k routed NVFP4 expert FFN
  moe_w4a16_gemv_trace         ... one token, with per-workgroup phase timestamps
  moe_layer_w4a16              router + routed experts + gated shared expert
  moe_workspace_status         sticky status of a MoE workspace (host query)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4_mtp.so")
_lib = None

NVFP4_OUT_F32 = 0
NVFP4_OUT_BF16 = 1
NVFP4_ARGMAX_BF16_KEYS = 1


class _Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_", ctypes.c_void_p),
                ("n", ctypes.c_int32), ("k", ctypes.c_int32)]


class _MoeWeights(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("gate_codes", ctypes.c_void_p), ("gate_scales", ctypes.c_void_p), ("gate_global", ctypes.c_void_p),
                ("up_codes", ctypes.c_void_p), ("up_scales", ctypes.c_void_p), ("up_global", ctypes.c_void_p),
                ("down_codes", ctypes.c_void_p), ("down_scales", ctypes.c_void_p), ("down_global", ctypes.c_void_p)]


class NVFP4Error(RuntimeError):
    pass


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NVFP4Error(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                             "or python nvfp4_w4a16_mtp_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        WP = ctypes.POINTER(_Weight)
        EP = ctypes.POINTER(_MoeWeights)
        L.nvfp4_quantize.argtypes = [P, i32, i32, P, P, P, P]
        L.w4a16_gemv.argtypes = [P, i32, WP, P, i32, P]
        L.w4a16_gemv_grouped.argtypes = [P, i32, ctypes.POINTER(WP), ctypes.POINTER(P), i32, i32, P]
        L.w4a16_gemm_m128_workspace_bytes.argtypes = [i32, i32, i32]
        L.w4a16_gemm_m128_workspace_bytes.restype = sz
        L.w4a16_gemm_m128.argtypes = [P, i32, WP, P, i32, P, sz, P]
        L.lmhead_gemv_argmax_workspace_bytes.argtypes = [i32, i32]
        L.lmhead_gemv_argmax_workspace_bytes.restype = sz
        L.lmhead_gemv_argmax.argtypes = [P, i32, WP, i32, P, P, P, sz, u32, P]
        L.lmhead_gemv_argmax_noalloc.argtypes = [P, i32, WP, i32, P, P, u32, P]
        L.lmhead_gemv_argmax_logprob.argtypes = [P, i32, WP, i32, P, P, P, P, sz, u32, P]
        L.lmhead_gemv_argmax_masked.argtypes = [P, i32, WP, i32, P, i32, P, P, P, P, sz, u32, P]
        L.embed_from_argmax.argtypes = [P, i32, P, i32, i32, P, ctypes.c_int64, P, P]
        L.w4a16_gemv_embed.argtypes = [P, P, i32, i32, P, i32, WP, P, i32, P]
        L.lmhead_gemv_argmax_embed.argtypes = [P, i32, WP, i32, P, i32, P, P, P, P, i32, i32, P, ctypes.c_int64, P,
                                               P, sz, u32, P]
        L.lmhead_gemv_argmax_fc.argtypes = [P, i32, WP, i32, P, P, P, sz, u32, P, i32, i32, P, WP, P, i32, P]
        L.moe_w4a16_gemv_workspace_bytes.argtypes = [i32, i32, EP]
        L.moe_w4a16_gemv_workspace_bytes.restype = sz
        L.moe_w4a16_gemv.argtypes = [P, i32, P, i32, EP, P, P, P, P, sz, P]
        L.moe_w4a16_gemv_trace_words.argtypes = [i32, i32, EP]
        L.moe_w4a16_gemv_trace_words.restype = sz
        L.moe_w4a16_gemv_trace.argtypes = [P, i32, P, i32, EP, P, P, P, P, sz, P, sz, P]
        L.moe_layer_w4a16_workspace_bytes.argtypes = [i32, i32, EP]
        L.moe_layer_w4a16_workspace_bytes.restype = sz
        L.moe_layer_w4a16.argtypes = [P, i32, WP, i32, EP, WP, WP, WP, P, P, P, P, P, P, sz, P]
        L.moe_workspace_status.argtypes = [P, sz, ctypes.POINTER(u32), P]
        L.nvfp4_mtp_last_error.restype = ctypes.c_char_p
        for f in ("nvfp4_quantize", "w4a16_gemv", "w4a16_gemv_grouped", "w4a16_gemm_m128", "lmhead_gemv_argmax",
                  "lmhead_gemv_argmax_noalloc",
                  "lmhead_gemv_argmax_logprob", "lmhead_gemv_argmax_masked", "embed_from_argmax", "lmhead_gemv_argmax_embed",
                  "lmhead_gemv_argmax_fc",
                  "w4a16_gemv_embed",
                  "moe_w4a16_gemv", "moe_w4a16_gemv_trace", "moe_layer_w4a16", "moe_workspace_status"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = lib().nvfp4_mtp_last_error().decode(errors="replace")
        raise NVFP4Error(f"{what} failed ({rc}): {msg}")


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _as_bf16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t.view(torch.bfloat16)
    raise TypeError(f"expected bf16 (or 16-bit bit patterns), got {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class NVFP4Weight:
    """One NVFP4 matrix W[n, k] on the device: codes [n, k/2] u8, scales
    [n, k/16] u8 (E4M3FN), glob 4 x fp32 = the 16-byte nvfp4_global struct
    {dec, enc, amax, flags}."""
    codes: torch.Tensor
    scales: torch.Tensor
    glob: torch.Tensor
    n: int
    k: int

    def desc(self) -> _Weight:
        return _Weight(self.codes.data_ptr(), self.scales.data_ptr(), self.glob.data_ptr(), self.n, self.k)

    @staticmethod
    def from_parts(codes: torch.Tensor, scales: torch.Tensor, g_dec: float) -> "NVFP4Weight":
        n, half = codes.shape
        glob = torch.tensor([float(g_dec), 0.0, 0.0, 0.0], dtype=torch.float32, device=codes.device)
        return NVFP4Weight(codes.contiguous(), scales.contiguous(), glob, n, half * 2)


@dataclass
class NVFP4Experts:
    """Stacked routed experts: gate/up codes [E, I, H/2], scales [E, I, H/16];
    down codes [E, H, I/2], scales [E, H, I/16]; globals [E, 4] fp32."""
    gate_codes: torch.Tensor
    gate_scales: torch.Tensor
    gate_glob: torch.Tensor
    up_codes: torch.Tensor
    up_scales: torch.Tensor
    up_glob: torch.Tensor
    down_codes: torch.Tensor
    down_scales: torch.Tensor
    down_glob: torch.Tensor

    @property
    def num_experts(self):
        return self.gate_codes.shape[0]

    @property
    def inter(self):
        return self.gate_codes.shape[1]

    @property
    def hidden(self):
        return self.gate_codes.shape[2] * 2

    def desc(self) -> _MoeWeights:
        return _MoeWeights(self.num_experts, self.hidden, self.inter,
                           self.gate_codes.data_ptr(), self.gate_scales.data_ptr(), self.gate_glob.data_ptr(),
                           self.up_codes.data_ptr(), self.up_scales.data_ptr(), self.up_glob.data_ptr(),
                           self.down_codes.data_ptr(), self.down_scales.data_ptr(), self.down_glob.data_ptr())


def nvfp4_quantize(w: torch.Tensor, out: NVFP4Weight | None = None) -> NVFP4Weight:
    w = _as_bf16(w)
    _dev(w, "w")
    n, k = w.shape
    if out is None:
        dev = w.device
        out = NVFP4Weight(torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                          torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
                          torch.empty(4, dtype=torch.float32, device=dev), n, k)
    _check(lib().nvfp4_quantize(_ptr(w), n, k, _ptr(out.codes), _ptr(out.scales), _ptr(out.glob), _stream(w)),
           "nvfp4_quantize")
    return out


def _out_code(dtype):
    if dtype == torch.float32:
        return NVFP4_OUT_F32
    if dtype == torch.bfloat16:
        return NVFP4_OUT_BF16
    raise TypeError("output dtype must be float32 or bfloat16")


def w4a16_gemv(x: torch.Tensor, w: NVFP4Weight, out_dtype=torch.float32, out: torch.Tensor | None = None):
    x = _as_bf16(x)
    _dev(x, "x")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.n), dtype=out_dtype, device=x.device)
    d = w.desc()
    _check(lib().w4a16_gemv(_ptr(x), m, ctypes.byref(d), _ptr(out), _out_code(out.dtype), _stream(x)), "w4a16_gemv")
    return out


def w4a16_gemv_embed(idx: torch.Tensor, table: torch.Tensor, x_rest: torch.Tensor | None, w: NVFP4Weight,
                     out_dtype=torch.float32, out: torch.Tensor | None = None):
    """w4a16_gemv over rows [table[idx[i]] | x_rest[i]]: the embedding rows
    of the tokens in idx (int32, e.g. the LM head's out_idx; zero rows for
    ids outside the table) are read by the GEMV itself."""
    _dev(idx, "idx")
    _dev(table, "table")
    if table.dtype != torch.bfloat16 or table.dim() != 2 or not table.is_contiguous():
        raise ValueError("table must be a contiguous bf16 [vocab][hidden] tensor")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    m = idx.numel()
    vocab, hidden = table.shape
    if x_rest is not None:
        x_rest = _as_bf16(x_rest)
        _dev(x_rest, "x_rest")
        if x_rest.shape != (m, w.k - hidden):
            raise ValueError(f"x_rest must be [{m}][{w.k - hidden}]")
    if out is None:
        out = torch.empty((m, w.n), dtype=out_dtype, device=table.device)
    d = w.desc()
    _check(lib().w4a16_gemv_embed(_ptr(idx), _ptr(table), vocab, hidden, _ptr(x_rest), m, ctypes.byref(d), _ptr(out),
                                  _out_code(out.dtype), _stream(table)), "w4a16_gemv_embed")
    return out


def w4a16_gemv_grouped(x: torch.Tensor, ws, out_dtype=torch.float32, outs=None):
    """One launch of the GEMV over several weights with the same K (q|k|v,
    gate|up); returns one output per weight."""
    x = _as_bf16(x)
    _dev(x, "x")
    m = x.shape[0]
    ws = list(ws)
    if outs is None:
        outs = [torch.empty((m, w.n), dtype=out_dtype, device=x.device) for w in ws]
    outs = list(outs)
    if len(outs) != len(ws):
        raise ValueError("w4a16_gemv_grouped: one output per weight")
    code = _out_code(outs[0].dtype) if outs else 0
    for o in outs:
        if _out_code(o.dtype) != code:
            raise ValueError("w4a16_gemv_grouped: all outputs need one dtype")
    descs = [w.desc() for w in ws]
    WP = ctypes.POINTER(_Weight)
    warr = (WP * len(ws))(*[ctypes.pointer(d) for d in descs])
    yarr = (ctypes.c_void_p * len(ws))(*[_ptr(o) for o in outs])
    _check(lib().w4a16_gemv_grouped(_ptr(x), m, warr, yarr, len(ws), code, _stream(x)), "w4a16_gemv_grouped")
    return outs


def gemm_workspace(m: int, n: int, k: int, device) -> torch.Tensor | None:
    """Workspace for w4a16_gemm_m128 at m x n x k on `device` (None when the
    call needs none: its output tiles fill the device)."""
    with torch.cuda.device(device):
        nbytes = lib().w4a16_gemm_m128_workspace_bytes(m, n, k)
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def w4a16_gemm_m128(x: torch.Tensor, w: NVFP4Weight, out_dtype=torch.float32, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, split_k: bool = True):
    """y = x @ W^T.  Short prompt chunks split K over a workspace (allocated
    here when none is given); split_k=False runs one pass over K."""
    x = _as_bf16(x)
    _dev(x, "x")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.n), dtype=out_dtype, device=x.device)
    if split_k and workspace is None:
        workspace = gemm_workspace(m, w.n, w.k, x.device)
    if not split_k:
        workspace = None
    if workspace is not None:
        _dev(workspace, "workspace")
    d = w.desc()
    _check(lib().w4a16_gemm_m128(_ptr(x), m, ctypes.byref(d), _ptr(out), _out_code(out.dtype),
                                 _ptr(workspace) if workspace is not None else None,
                                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                 _stream(x)), "w4a16_gemm_m128")
    return out


def lmhead_workspace(m: int, vocab_rows: int, device) -> torch.Tensor:
    """Zero-filled workspace for lmhead_gemv_argmax scoring `vocab_rows` rows
    (the effective V).  It must start zeroed; every call leaves it reusable."""
    nbytes = lib().lmhead_gemv_argmax_workspace_bytes(m, vocab_rows)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def lmhead_gemv_argmax(h: torch.Tensor, w: NVFP4Weight, vocab_rows: int = 0, bf16_keys: bool = False,
                       workspace: torch.Tensor | None = None, out_idx: torch.Tensor | None = None,
                       out_max: torch.Tensor | None = None):
    h = _as_bf16(h)
    _dev(h, "h")
    m = h.shape[0]
    if workspace is None:
        v = w.n if vocab_rows <= 0 else min(vocab_rows, w.n)
        workspace = lmhead_workspace(m, v, h.device)
    if out_idx is None:
        out_idx = torch.empty(m, dtype=torch.int32, device=h.device)
    if out_max is None:
        out_max = torch.empty(m, dtype=torch.float32, device=h.device)
    d = w.desc()
    _check(lib().lmhead_gemv_argmax(_ptr(h), m, ctypes.byref(d), vocab_rows, _ptr(out_idx), _ptr(out_max),
                                    _ptr(workspace), workspace.numel(),
                                    NVFP4_ARGMAX_BF16_KEYS if bf16_keys else 0, _stream(h)),
           "lmhead_gemv_argmax")
    return out_idx, out_max


def lmhead_gemv_argmax_fc(h: torch.Tensor, w: NVFP4Weight, table: torch.Tensor, x_rest: torch.Tensor | None,
                          fc: NVFP4Weight, vocab_rows: int = 0, bf16_keys: bool = False,
                          workspace: torch.Tensor | None = None, out_idx: torch.Tensor | None = None,
                          out_max: torch.Tensor | None = None, out: torch.Tensor | None = None,
                          out_dtype=torch.float32):
    """lmhead_gemv_argmax of h, then the next draft step's fc over the rows
    [table[out_idx[i]] | x_rest[i]] (w4a16_gemv_embed): one launch at one
    row, the two calls otherwise.  Returns (out_idx, out_max, out)."""
    h = _as_bf16(h)
    _dev(h, "h")
    _dev(table, "table")
    if table.dtype != torch.bfloat16 or table.dim() != 2 or not table.is_contiguous():
        raise ValueError("table must be a contiguous bf16 [vocab][hidden] tensor")
    m = h.shape[0]
    vocab, hidden = table.shape
    if x_rest is not None:
        x_rest = _as_bf16(x_rest)
        _dev(x_rest, "x_rest")
        if x_rest.shape != (m, fc.k - hidden):
            raise ValueError(f"x_rest must be [{m}][{fc.k - hidden}]")
    if workspace is None:
        v = w.n if vocab_rows <= 0 else min(vocab_rows, w.n)
        workspace = lmhead_workspace(m, v, h.device)
    if out_idx is None:
        out_idx = torch.empty(m, dtype=torch.int32, device=h.device)
    if out_max is None:
        out_max = torch.empty(m, dtype=torch.float32, device=h.device)
    if out is None:
        out = torch.empty((m, fc.n), dtype=out_dtype, device=h.device)
    d, dfc = w.desc(), fc.desc()
    _check(lib().lmhead_gemv_argmax_fc(_ptr(h), m, ctypes.byref(d), vocab_rows, _ptr(out_idx), _ptr(out_max),
                                       _ptr(workspace), workspace.numel(), NVFP4_ARGMAX_BF16_KEYS if bf16_keys else 0,
                                       _ptr(table), vocab, hidden, _ptr(x_rest), ctypes.byref(dfc), _ptr(out),
                                       _out_code(out.dtype), _stream(h)),
           "lmhead_gemv_argmax_fc")
    return out_idx, out_max, out


def lmhead_gemv_argmax_noalloc(h: torch.Tensor, w: NVFP4Weight, vocab_rows: int = 0, bf16_keys: bool = False,
                               out_idx: torch.Tensor | None = None, out_max: torch.Tensor | None = None):
    """lmhead_gemv_argmax with the library's static per-device scratch in
    place of a workspace (nothing is allocated by the call itself; pass
    out_idx / out_max to allocate nothing here either).  Calls that overlap
    on one device race."""
    h = _as_bf16(h)
    _dev(h, "h")
    m = h.shape[0]
    if out_idx is None:
        out_idx = torch.empty(m, dtype=torch.int32, device=h.device)
    if out_max is None:
        out_max = torch.empty(m, dtype=torch.float32, device=h.device)
    d = w.desc()
    _check(lib().lmhead_gemv_argmax_noalloc(_ptr(h), m, ctypes.byref(d), vocab_rows, _ptr(out_idx), _ptr(out_max),
                                            NVFP4_ARGMAX_BF16_KEYS if bf16_keys else 0, _stream(h)),
           "lmhead_gemv_argmax_noalloc")
    return out_idx, out_max


def lmhead_gemv_argmax_logprob(h: torch.Tensor, w: NVFP4Weight, vocab_rows: int = 0, bf16_keys: bool = False,
                               workspace: torch.Tensor | None = None, out_idx: torch.Tensor | None = None,
                               out_max: torch.Tensor | None = None, out_logprob: torch.Tensor | None = None):
    """lmhead_gemv_argmax plus the top-1 log-probability of each selected token."""
    h = _as_bf16(h)
    _dev(h, "h")
    m = h.shape[0]
    if workspace is None:
        v = w.n if vocab_rows <= 0 else min(vocab_rows, w.n)
        workspace = lmhead_workspace(m, v, h.device)
    if out_idx is None:
        out_idx = torch.empty(m, dtype=torch.int32, device=h.device)
    if out_max is None:
        out_max = torch.empty(m, dtype=torch.float32, device=h.device)
    if out_logprob is None:
        out_logprob = torch.empty(m, dtype=torch.float32, device=h.device)
    d = w.desc()
    _check(lib().lmhead_gemv_argmax_logprob(_ptr(h), m, ctypes.byref(d), vocab_rows, _ptr(out_idx), _ptr(out_max),
                                            _ptr(out_logprob), _ptr(workspace), workspace.numel(),
                                            NVFP4_ARGMAX_BF16_KEYS if bf16_keys else 0, _stream(h)),
           "lmhead_gemv_argmax_logprob")
    return out_idx, out_max, out_logprob


def lmhead_gemv_argmax_masked(h: torch.Tensor, w: NVFP4Weight, allow_mask: torch.Tensor, vocab_rows: int = 0,
                              bf16_keys: bool = False, with_logprob: bool = False,
                              workspace: torch.Tensor | None = None, out_idx: torch.Tensor | None = None,
                              out_max: torch.Tensor | None = None, out_logprob: torch.Tensor | None = None):
    """Grammar-masked LM-head argmax.  allow_mask: int32/uint32 [m][words] on
    the device (bit r % 32 of word r / 32 allows token r)."""
    h = _as_bf16(h)
    _dev(h, "h")
    _dev(allow_mask, "allow_mask")
    m = h.shape[0]
    if allow_mask.dim() != 2 or allow_mask.shape[0] != m or allow_mask.element_size() != 4:
        raise ValueError("allow_mask must be a [m][words] 32-bit tensor")
    allow_mask = allow_mask.contiguous()
    if workspace is None:
        v = w.n if vocab_rows <= 0 else min(vocab_rows, w.n)
        workspace = lmhead_workspace(m, v, h.device)
    if out_idx is None:
        out_idx = torch.empty(m, dtype=torch.int32, device=h.device)
    if out_max is None:
        out_max = torch.empty(m, dtype=torch.float32, device=h.device)
    if with_logprob and out_logprob is None:
        out_logprob = torch.empty(m, dtype=torch.float32, device=h.device)
    d = w.desc()
    _check(lib().lmhead_gemv_argmax_masked(_ptr(h), m, ctypes.byref(d), vocab_rows, _ptr(allow_mask),
                                           allow_mask.shape[1], _ptr(out_idx), _ptr(out_max), _ptr(out_logprob),
                                           _ptr(workspace), workspace.numel(),
                                           NVFP4_ARGMAX_BF16_KEYS if bf16_keys else 0, _stream(h)),
           "lmhead_gemv_argmax_masked")
    return (out_idx, out_max, out_logprob) if with_logprob else (out_idx, out_max)


def embed_from_argmax(idx: torch.Tensor, table: torch.Tensor, out: torch.Tensor | None = None,
                      id_log: torch.Tensor | None = None):
    """Rows table[idx[i]] of a bf16 [vocab][hidden] table (zero rows for
    out-of-range ids) into out (rows may be strided, e.g. half of a wider
    activation row); id_log, if given, receives the ids."""
    _dev(idx, "idx")
    _dev(table, "table")
    if table.dtype != torch.bfloat16 or table.dim() != 2 or not table.is_contiguous():
        raise ValueError("table must be a contiguous bf16 [vocab][hidden] tensor")
    m = idx.numel()
    vocab, hidden = table.shape
    if out is None:
        out = torch.empty((m, hidden), dtype=torch.bfloat16, device=table.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.shape[1] != hidden or out.stride(1) != 1:
        raise ValueError("out must be bf16 [m][hidden] with unit column stride")
    _check(lib().embed_from_argmax(_ptr(idx), m, _ptr(table), vocab, hidden, _ptr(out), out.stride(0), _ptr(id_log),
                                   _stream(table)), "embed_from_argmax")
    return out


def lmhead_gemv_argmax_embed(h: torch.Tensor, w: NVFP4Weight, table: torch.Tensor, out_embed: torch.Tensor,
                             vocab_rows: int = 0, allow_mask: torch.Tensor | None = None, bf16_keys: bool = False,
                             id_log: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                             out_idx: torch.Tensor | None = None, out_max: torch.Tensor | None = None,
                             out_logprob: torch.Tensor | None = None):
    """LM-head argmax whose last workgroup also writes table[idx[i]] into
    out_embed row i (bf16, unit column stride) and idx into id_log."""
    h = _as_bf16(h)
    _dev(h, "h")
    _dev(table, "table")
    m = h.shape[0]
    if table.dtype != torch.bfloat16 or table.dim() != 2 or not table.is_contiguous():
        raise ValueError("table must be a contiguous bf16 [vocab][hidden] tensor")
    vocab, hidden = table.shape
    if out_embed.dtype != torch.bfloat16 or out_embed.dim() != 2 or out_embed.shape != (m, hidden) \
            or out_embed.stride(1) != 1:
        raise ValueError("out_embed must be bf16 [m][hidden] with unit column stride")
    words = 0
    if allow_mask is not None:
        _dev(allow_mask, "allow_mask")
        allow_mask = allow_mask.contiguous()
        words = allow_mask.shape[1]
    if workspace is None:
        v = w.n if vocab_rows <= 0 else min(vocab_rows, w.n)
        workspace = lmhead_workspace(m, v, h.device)
    if out_idx is None:
        out_idx = torch.empty(m, dtype=torch.int32, device=h.device)
    if out_max is None:
        out_max = torch.empty(m, dtype=torch.float32, device=h.device)
    d = w.desc()
    _check(lib().lmhead_gemv_argmax_embed(_ptr(h), m, ctypes.byref(d), vocab_rows, _ptr(allow_mask), words,
                                          _ptr(out_idx), _ptr(out_max), _ptr(out_logprob), _ptr(table), vocab, hidden,
                                          _ptr(out_embed), out_embed.stride(0), _ptr(id_log), _ptr(workspace),
                                          workspace.numel(), NVFP4_ARGMAX_BF16_KEYS if bf16_keys else 0, _stream(h)),
           "lmhead_gemv_argmax_embed")
    return out_idx, out_max


def moe_workspace(m: int, top_k: int, experts: NVFP4Experts, device) -> torch.Tensor:
    """Zero-filled workspace for moe_w4a16_gemv (must start zeroed; every call
    leaves it reusable)."""
    d = experts.desc()
    nbytes = lib().moe_w4a16_gemv_workspace_bytes(m, top_k, ctypes.byref(d))
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def moe_trace_events(top_k: int, experts: NVFP4Experts) -> tuple[int, int]:
    """(events, workgroups) of a one-token moe_w4a16_gemv_trace: the trace
    holds events x workgroups timestamps, gate/up workgroups first."""
    d = experts.desc()
    words = lib().moe_w4a16_gemv_trace_words(1, top_k, ctypes.byref(d))
    return 6, words // 6


def moe_w4a16_gemv(x: torch.Tensor, router_logits: torch.Tensor, top_k: int, experts: NVFP4Experts,
                   workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                   trace: torch.Tensor | None = None):
    """Routed MoE over m rows.  With `trace` (int64 [6, workgroups] from
    moe_trace_events, one token only) the one-launch form also records its
    phase timestamps (moe_w4a16_gemv_trace)."""
    x = _as_bf16(x)
    _dev(x, "x")
    _dev(router_logits, "router_logits")
    if router_logits.dtype != torch.float32:
        raise TypeError("router_logits must be float32")
    m = x.shape[0]
    if workspace is None:
        workspace = moe_workspace(m, top_k, experts, x.device)
    if out is None:
        out = torch.empty((m, experts.hidden), dtype=torch.float32, device=x.device)
    if topk_ids is None:
        topk_ids = torch.empty((m, top_k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((m, top_k), dtype=torch.float32, device=x.device)
    d = experts.desc()
    if trace is not None:
        _dev(trace, "trace")
        if trace.dtype != torch.int64 or not trace.is_contiguous():
            raise TypeError("trace must be a contiguous int64 tensor")
        _check(lib().moe_w4a16_gemv_trace(_ptr(x), m, _ptr(router_logits), top_k, ctypes.byref(d), _ptr(out),
                                          _ptr(topk_ids), _ptr(topk_w), _ptr(workspace), workspace.numel(),
                                          _ptr(trace), trace.numel(), _stream(x)),
               "moe_w4a16_gemv_trace")
        return out, topk_ids, topk_w
    _check(lib().moe_w4a16_gemv(_ptr(x), m, _ptr(router_logits), top_k, ctypes.byref(d), _ptr(out), _ptr(topk_ids),
                                _ptr(topk_w), _ptr(workspace), workspace.numel(), _stream(x)),
           "moe_w4a16_gemv")
    return out, topk_ids, topk_w


def moe_workspace_status(workspace: torch.Tensor) -> int:
    """Reads and clears the sticky status word of a MoE workspace
    (synchronizes the current stream).  Returns 0; raises NVFP4Error when a
    down pass gave up its wait or found the workspace overwritten."""
    _dev(workspace, "workspace")
    st = ctypes.c_uint32(0)
    _check(lib().moe_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                      ctypes.byref(st), _stream(workspace)), "moe_workspace_status")
    return st.value


def moe_layer_workspace(m: int, top_k: int, experts: NVFP4Experts, device) -> torch.Tensor:
    """Zero-filled workspace for moe_layer_w4a16."""
    d = experts.desc()
    nbytes = lib().moe_layer_w4a16_workspace_bytes(m, top_k, ctypes.byref(d))
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def moe_layer_w4a16(x: torch.Tensor, router: NVFP4Weight, top_k: int, experts: NVFP4Experts,
                    shared_gate: NVFP4Weight, shared_up: NVFP4Weight, shared_down: NVFP4Weight,
                    shared_gate_w: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, topk_ids: torch.Tensor | None = None,
                    topk_w: torch.Tensor | None = None, router_logits: torch.Tensor | None = None):
    """The complete MoE layer; returns (y, topk_ids, topk_w, router_logits)."""
    x = _as_bf16(x)
    _dev(x, "x")
    m = x.shape[0]
    dev = x.device
    if workspace is None:
        workspace = moe_layer_workspace(m, top_k, experts, dev)
    if out is None:
        out = torch.empty((m, experts.hidden), dtype=torch.float32, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty((m, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((m, top_k), dtype=torch.float32, device=dev)
    if router_logits is None:
        router_logits = torch.empty((m, experts.num_experts), dtype=torch.float32, device=dev)
    if shared_gate_w is not None:
        shared_gate_w = _as_bf16(shared_gate_w).contiguous()
    ds = [w.desc() for w in (router, shared_gate, shared_up, shared_down)]
    d = experts.desc()
    _check(lib().moe_layer_w4a16(_ptr(x), m, ctypes.byref(ds[0]), top_k, ctypes.byref(d), ctypes.byref(ds[1]),
                                 ctypes.byref(ds[2]), ctypes.byref(ds[3]), _ptr(shared_gate_w), _ptr(out),
                                 _ptr(topk_ids), _ptr(topk_w), _ptr(router_logits), _ptr(workspace),
                                 workspace.numel(), _stream(x)), "moe_layer_w4a16")
    return out, topk_ids, topk_w, router_logits

