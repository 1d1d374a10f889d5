"""The HIP library loads on a machine without a GPU and exports every
function include/nvfp4_mtp.h declares (no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_mtp.h")
LIB = os.path.join(ROOT, "nvfp4_w4a16_mtp_amd", "libnvfp4_mtp.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(", src, re.M)
    return sorted(set(names))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for f in ("nvfp4_quantize", "w4a16_gemv", "w4a16_gemv_grouped", "w4a16_gemm_m128", "lmhead_gemv_argmax", "lmhead_gemv_argmax_logprob", "lmhead_gemv_argmax_masked", "embed_from_argmax", "lmhead_gemv_argmax_embed", "lmhead_gemv_argmax_fc", "w4a16_gemv_embed", "moe_w4a16_gemv", "moe_layer_w4a16",
              "moe_workspace_status", "moe_w4a16_gemv_trace", "moe_w4a16_gemv_trace_words", "lmhead_gemv_argmax_noalloc", "lmhead_gemv_argmax_workspace_bytes", "moe_w4a16_gemv_workspace_bytes", "w4a16_gemm_m128_workspace_bytes",
              "nvfp4_mtp_last_error"):
        assert f in names, f


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built (run __graft_entry__.build())")
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(LIB)
    for f in declared_functions():
        assert hasattr(L, f), f"{f} declared in nvfp4_mtp.h but not exported"


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built (run __graft_entry__.build())")
def test_argument_errors_need_no_gpu():
    """Host-side validation rejects bad arguments before touching the GPU."""
    import nvfp4_w4a16_mtp_amd as nv
    L = nv.lib()
    w = nv._Weight(0, 0, 0, 16, 32)
    assert L.w4a16_gemv(None, 1, ctypes.byref(w), None, 0, None) == -1
    assert b"NULL" in L.nvfp4_mtp_last_error()
    assert L.nvfp4_quantize(ctypes.c_void_p(16), 4, 48, ctypes.c_void_p(16), ctypes.c_void_p(16),
                            ctypes.c_void_p(16), None) == -2
    assert L.lmhead_gemv_argmax_workspace_bytes(8, 151936) >= 8 * 16
    ok_ptr = ctypes.c_void_p(256)
    assert L.w4a16_gemv_embed(None, ok_ptr, 10, 32, ok_ptr, 1, ctypes.byref(w), ok_ptr, 0, None) == -1
    assert L.w4a16_gemv_embed(ok_ptr, ok_ptr, 10, 40, ok_ptr, 1, ctypes.byref(w), ok_ptr, 0, None) == -2
    assert b"hidden" in L.nvfp4_mtp_last_error()
    st = ctypes.c_uint32(7)
    assert L.moe_workspace_status(None, 1 << 20, ctypes.byref(st), None) == -1
    assert L.moe_workspace_status(ctypes.c_void_p(256), 64, ctypes.byref(st), None) == -4
    assert st.value == 7
