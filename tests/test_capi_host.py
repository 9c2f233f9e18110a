"""The C-ABI library loads, exports every function include/nvfp4moe.h
declares, and rejects invalid arguments on the host before any HIP call (no
GPU needed: these calls return before touching the device)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")
LIB = os.path.join(ROOT, "nvfp4_w4a4_quantized_amd", "libnvfp4moe.so")
DEBUG_LIB = os.path.join(ROOT, "nvfp4_w4a4_quantized_amd", "libnvfp4moe_debug.so")

INVALID, UNSUPPORTED, WS_SMALL = 1, 2, 4


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "sizeof")))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    from nvfp4_w4a4_quantized_amd import _lib
    return _lib.lib()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("nvfp4_quantize", "moe_permute", "w4a4_grouped_gemm", "w4a4_grouped_gemm_swiglu",
              "moe_combine", "moe_expert_forward", "moe_rows_capacity",
              "moe_permute_workspace_size", "moe_expert_forward_workspace_size",
              "nvfp4_status_string", "nvfp4_pack_weights"):
        assert n in names


@pytest.mark.parametrize("path", [LIB, DEBUG_LIB], ids=["release", "debug"])
def test_library_exports_every_declared_symbol(path):
    if not os.path.exists(path):
        pytest.fail(f"{path} not built (run __graft_entry__.build())")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    lib = C.CDLL(path)
    for n in _declared_functions():
        getattr(lib, n)   # resolvable through ctypes


def test_debug_build_reports_itself(L):
    """The precondition checks exist only in the NVFP4_DEBUG_CHECKS build."""
    from nvfp4_w4a4_quantized_amd import _lib
    assert L.nvfp4_debug_checks() == 0
    assert _lib.debug_lib().nvfp4_debug_checks() == 1
    # both builds reserve the same workspace (the word's slot included)
    for args in ((8192, 8, 128), (1, 1, 1), (32768, 8, 1024)):
        assert L.moe_permute_workspace_size(*args) == _lib.debug_lib().moe_permute_workspace_size(*args)


def test_host_side_sizes(L):
    assert L.moe_rows_capacity(8192, 8, 128, 1) == 65536
    assert L.moe_rows_capacity(100, 4, 7, 16) == 100 * 4 + 7 * 15
    assert L.moe_permute_workspace_size(8192, 8, 128) >= 128 * 128 * 4
    ws = L.moe_expert_forward_workspace_size(8192, 2048, 768, 8, 128, 1)
    cap = 65536
    # token-major quantized activations, D, A2 and the FC2 rows
    assert ws >= 8192 * (2048 // 2 + 2048 // 16) + cap * (768 * 2 + 768 // 2 + 768 // 16 + 2048 * 2)
    assert L.nvfp4_status_string(0) == b"ok"
    assert L.nvfp4_status_string(4) == b"workspace too small"


def test_invalid_arguments_rejected_before_any_device_call(L):
    fake = C.c_void_p(0x1000)   # never dereferenced: validation fails first
    # k not a multiple of 16
    assert L.nvfp4_quantize(fake, 4, 24, 24, 0, None, 0, None, 0, fake, fake, fake, None) == INVALID
    # missing output
    assert L.nvfp4_quantize(fake, 4, 32, 32, 0, None, 0, None, 0, None, fake, fake, None) == INVALID
    # unknown domain / domain 1 without offsets
    assert L.nvfp4_quantize(fake, 4, 32, 32, 1, None, 2, None, 0, fake, fake, fake, None) == INVALID
    # k beyond the supported maximum
    assert L.nvfp4_quantize(fake, 4, 32768, 32768, 0, None, 0, None, 0, fake, fake, fake, None) == UNSUPPORTED
    # 16x16 blocks need rows % 16 == 0 and the standard rule
    assert L.nvfp4_quantize(fake, 24, 32, 32, 2, fake, 1, None, 0, fake, fake, fake, None) == UNSUPPORTED
    assert L.nvfp4_quantize(fake, 32, 32, 32, 2, fake, 1, None, 1, fake, fake, fake, None) == UNSUPPORTED
    # unknown block rule
    assert L.nvfp4_quantize(fake, 4, 32, 32, 0, None, 0, None, 3, fake, fake, fake, None) == INVALID
    # misaligned x
    assert L.nvfp4_quantize(C.c_void_p(0x1002), 4, 32, 32, 0, None, 0, None, 0, fake, fake, fake, None) == INVALID
    # topk > experts, bad align, too many experts
    args = (fake, 16, 64, fake, fake)
    assert L.moe_permute(*args, 5, 4, 1, 0, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 20, None) == INVALID
    assert L.moe_permute(*args, 2, 4, 3, 0, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 20, None) == INVALID
    assert L.moe_permute(*args, 2, 2048, 1, 0, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 20, None) == INVALID
    # workspace too small
    assert L.moe_permute(*args, 2, 4, 1, 0, fake, fake, fake, fake, fake, fake, fake, fake, 4, None) == WS_SMALL
    assert L.moe_permute(*args, 2, 4, 1, 7, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 20, None) == INVALID
    # GEMM: k not a multiple of 128, n not a multiple of 32, bad dtype
    g = (fake, fake, fake, 64, fake, fake, fake, fake, 2)
    assert L.w4a4_grouped_gemm(*g, 64, 96, 0, 0, fake, None) == UNSUPPORTED
    assert L.w4a4_grouped_gemm(*g, 48, 128, 0, 0, fake, None) == UNSUPPORTED
    assert L.w4a4_grouped_gemm(*g, 64, 128, 0, 7, fake, None) == INVALID
    assert L.w4a4_grouped_gemm(*g, 64, 128, 0, 1, C.c_void_p(0x1008), None) == INVALID   # out not 16-byte aligned
    assert L.w4a4_grouped_gemm(*g, 64, 120, 0, 0, fake, None) == INVALID
    # unknown B layout
    assert L.w4a4_grouped_gemm(*g, 64, 128, 2, 0, fake, None) == INVALID
    assert L.w4a4_grouped_gemm_swiglu(*g, 64, 128, 5, fake, fake, fake, None, None) == INVALID
    assert L.w4a4_grouped_gemm_swiglu(*g, 96, 128, 0, fake, fake, fake, None, None) == UNSUPPORTED
    # weight packing: n not a multiple of 32, k not a multiple of 128, missing output
    assert L.nvfp4_pack_weights(fake, fake, 2, 48, 128, fake, fake, None) == UNSUPPORTED
    assert L.nvfp4_pack_weights(fake, fake, 2, 64, 96, fake, fake, None) == UNSUPPORTED
    assert L.nvfp4_pack_weights(fake, fake, 2, 64, 128, None, fake, None) == INVALID
    # one group's B codes of 4 GiB or more (32-bit offsets inside a group)
    g1 = (fake, fake, fake, 64, fake, fake, fake, fake, 1)
    assert L.w4a4_grouped_gemm(*g1, 1 << 20, 8192, 0, 0, fake, None) == UNSUPPORTED
    assert L.w4a4_grouped_gemm_swiglu(*g1, 1 << 19, 8192, 0, fake, fake, fake, None, None) == UNSUPPORTED
    # combine: hidden not a multiple of 8
    assert L.moe_combine(fake, 0, fake, 4, 2, 12, fake, None) == INVALID
    # expert layer: hidden not a multiple of 128, missing weights
    from nvfp4_w4a4_quantized_amd._lib import Weights
    w = Weights(0x1000, 0x1000, 0x1000)
    assert L.moe_expert_forward(fake, 8, 200, 128, fake, fake, 2, 4, 1, 0, 0, C.byref(w), C.byref(w),
                                fake, C.c_void_p(0x10000), 1 << 30, None, None, None) == UNSUPPORTED
    assert L.moe_expert_forward(fake, 8, 256, 128, fake, fake, 2, 4, 1, 0, 0, None, C.byref(w),
                                fake, C.c_void_p(0x10000), 1 << 30, None, None, None) == INVALID
    assert L.moe_expert_forward(fake, 8, 256, 128, fake, fake, 2, 4, 1, 0, 0, C.byref(w),
                                C.byref(w), fake, C.c_void_p(0x10000), 16, None, None,
                                None) == WS_SMALL
    # unknown activation block rule, unknown activation scale domain
    assert L.moe_expert_forward(fake, 8, 256, 128, fake, fake, 2, 4, 1, 5, 0, C.byref(w),
                                C.byref(w), fake, C.c_void_p(0x10000), 1 << 30, None, None,
                                None) == INVALID
    assert L.moe_expert_forward(fake, 8, 256, 128, fake, fake, 2, 4, 1, 0, 2, C.byref(w),
                                C.byref(w), fake, C.c_void_p(0x10000), 1 << 30, None, None,
                                None) == INVALID
    wbad = Weights(0x1000, 0x1000, 0x1000, 3)   # unknown layout
    assert L.moe_expert_forward(fake, 8, 256, 128, fake, fake, 2, 4, 1, 0, 0, C.byref(w),
                                C.byref(wbad), fake, C.c_void_p(0x10000), 1 << 30, None, None,
                                None) == INVALID
    # backward: hidden not a multiple of 128, dw1 / dw2 not 16-byte aligned (the
    # weight-gradient tiles are stored in 16-byte pieces), workspace too small
    ws = C.c_void_p(0x10000)

    def bwd(hidden=256, dw1=fake, dw2=fake, ws_bytes=1 << 30):
        return L.moe_expert_backward(fake, fake, 8, hidden, 128, 2, 4, 64, fake, fake, fake, fake,
                                     fake, fake, fake, fake, fake, dw1, dw2, fake, ws, ws_bytes,
                                     None, None, None)
    assert bwd(hidden=200) == UNSUPPORTED
    assert bwd(dw1=C.c_void_p(0x1004)) == INVALID
    assert bwd(dw2=C.c_void_p(0x1008)) == INVALID
    assert bwd(ws_bytes=16) == WS_SMALL


def test_noalloc_permute_rejects_before_any_device_call(L):
    """moe_permute_noalloc checks its arguments and the scratch limit on the
    host, before its first HIP call (so these run without a GPU)."""
    SCRATCH_LIMIT = 5
    assert L.nvfp4_status_string(SCRATCH_LIMIT).startswith(b"exceeds the static scratch")
    limit = 4 << 20
    fake = C.c_void_p(0x1000)
    args = (fake, fake, fake, fake, fake, fake, fake, None)
    # the largest token counts that fit, and the first that do not
    for E, T_ok in ((128, 261_000), (1024, 32_700)):
        assert L.moe_permute_workspace_size(T_ok, 8, E) <= limit
        T_bad = T_ok
        while L.moe_permute_workspace_size(T_bad, 8, E) <= limit:
            T_bad += 64
        assert L.moe_permute_noalloc(fake, T_bad, 256, fake, fake, 8, E, 1, 0, *args) == SCRATCH_LIMIT
    # argument errors take precedence over the size
    assert L.moe_permute_noalloc(fake, 1 << 20, 256, fake, fake, 8, 1024, 3, 0, *args) == INVALID
    assert L.moe_permute_noalloc(fake, 16, 64, fake, fake, 5, 4, 1, 0, *args) == INVALID
    assert L.moe_permute_noalloc(fake, 16, 64, fake, fake, 2, 4, 1, 7, *args) == INVALID
    assert L.moe_permute_noalloc(fake, 16, 32768, fake, fake, 2, 4, 1, 0, *args) == UNSUPPORTED
