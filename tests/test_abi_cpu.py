"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects malformed calls before launching anything."""

import ctypes
import os
import subprocess

import pytest

import mxfp4_routed_expert_softmax_amd as M
from mxfp4_routed_expert_softmax_amd import _lib as L

FAKE = 0x10000  # an aligned non-null address; validation never dereferences it


def test_library_exports_every_header_function():
    names = M.header_functions()
    assert set(names) == {"moe_router_topk", "moe_permute", "moe_expert_ffn_mxfp4",
                          "moe_combine", "moe_layer_forward", "moe_workspace_bytes",
                          "moe_status_str", "moe_set_kernel_events",
                          "moe_last_call_launches", "moe_launch_name",
                          "moe_quantize_mxfp8", "moe_layer_forward_mxfp8_act",
                          "moe_expert_ffn_fp8", "moe_layer_forward_fp8_shared",
                          "moe_expert_ffn_nvfp4", "moe_layer_forward_nvfp4",
                          "moe_workspace_status", "moe_set_wait_test",
                          "moe_layer_forward_noalloc"}
    lib = M.lib()
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    assert set(names) <= exported


def test_status_strings():
    assert M.status_str(0) == "MOE_OK"
    assert M.status_str(-3) == "MOE_ERR_WORKSPACE"
    assert M.status_str(-5) == "MOE_ERR_TIMEOUT"
    assert M.status_str(99) == "MOE_ERR_UNKNOWN"


def test_workspace_bytes_grows_with_the_problem():
    a = M.moe_workspace_bytes(1, 5120, 2304, 384, 6)
    b = M.moe_workspace_bytes(16384, 5120, 2304, 384, 6)
    assert 0 < a < b
    # holds at least the fp32 routed rows and hidden activations of prefill
    assert b >= 16384 * 6 * (5120 + 2304) * 4
    assert M.moe_workspace_bytes(-1, 5120, 2304, 384, 6) == 0


def _bank(E=16, H=256, I=128, codes=FAKE):
    return L.Bank(codes, FAKE, FAKE, FAKE, E, H, I)


def _fwd(bank, shared=None, T=8, k=2, out=FAKE, ws=FAKE, ws_bytes=1 << 40, x=FAKE):
    lib = M.lib()
    return lib.moe_layer_forward(x, FAKE, None, ctypes.byref(bank),
                                 None if shared is None else ctypes.byref(shared),
                                 T, k, out, None, None, ws, ws_bytes, None)


def test_layer_forward_validation_codes():
    assert _fwd(_bank(), x=None) == M.MOE_ERR_INVALID_ARG
    assert _fwd(_bank(), out=None) == M.MOE_ERR_INVALID_ARG
    assert _fwd(_bank(codes=FAKE + 4)) == M.MOE_ERR_INVALID_ARG          # misaligned codes
    assert _fwd(_bank(H=250)) == M.MOE_ERR_INVALID_ARG                    # H % 32
    assert _fwd(_bank(I=100)) == M.MOE_ERR_INVALID_ARG                    # I % 32
    assert _fwd(_bank(), k=17) == M.MOE_ERR_INVALID_ARG                   # k > E
    assert _fwd(_bank(), T=-1) == M.MOE_ERR_INVALID_ARG
    assert _fwd(_bank(E=2048)) == M.MOE_ERR_UNSUPPORTED
    assert _fwd(_bank(E=128), k=65) == M.MOE_ERR_UNSUPPORTED
    assert _fwd(_bank(H=16384)) == M.MOE_ERR_UNSUPPORTED
    assert _fwd(_bank(), shared=_bank(E=2)) == M.MOE_ERR_INVALID_ARG      # shared must be E=1
    assert _fwd(_bank(), shared=_bank(E=1, I=64)) == M.MOE_ERR_INVALID_ARG
    assert _fwd(_bank(), ws_bytes=100) == M.MOE_ERR_WORKSPACE
    assert _fwd(_bank(), T=64, ws_bytes=M.moe_workspace_bytes(64, 256, 128, 16, 2) // 2) \
        == M.MOE_ERR_WORKSPACE
    assert _fwd(_bank(), ws=None) == M.MOE_ERR_INVALID_ARG
    assert _fwd(_bank(), T=0) == M.MOE_OK                                  # no-op


def test_other_calls_validate_before_launch():
    lib = M.lib()
    ok = lib.moe_router_topk(FAKE, FAKE, None, 0, 256, 16, 2, FAKE, FAKE, FAKE, None, 0, None)
    assert ok == M.MOE_OK
    assert lib.moe_router_topk(FAKE, FAKE, None, 4, 256, 16, 2, FAKE, FAKE, None, None, 0,
                               None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_router_topk(FAKE, FAKE, None, 4, 256, 16, 2, FAKE, FAKE, None, FAKE, 16,
                               None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_router_topk(FAKE + 2, FAKE, None, 4, 256, 16, 2, FAKE, FAKE, FAKE, None, 0,
                               None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(FAKE, 4, 2, 16, FAKE, FAKE, FAKE, None, 0, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(FAKE, 4, 2, 16, FAKE, FAKE, FAKE, FAKE, 8, None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_permute(FAKE, 0, 2, 16, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == M.MOE_OK
    b = _bank()
    assert lib.moe_expert_ffn_mxfp4(FAKE, ctypes.byref(b), None, None, 8, 16, FAKE, FAKE,
                                    1 << 30, None) == M.MOE_ERR_INVALID_ARG   # offsets needed
    b1 = _bank(E=1)
    assert lib.moe_expert_ffn_mxfp4(FAKE, ctypes.byref(b1), None, None, 8, 9, FAKE, FAKE,
                                    1 << 30, None) == M.MOE_ERR_INVALID_ARG   # R > T, no row_token
    assert lib.moe_expert_ffn_mxfp4(FAKE, ctypes.byref(b1), None, None, 8, 8, FAKE, FAKE,
                                    100, None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_combine(FAKE, None, FAKE, None, 4, 2, 256, 8, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(FAKE, FAKE, FAKE, None, 4, 2, 250, 8, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(FAKE, FAKE, FAKE, None, 0, 2, 256, 8, FAKE, None) == M.MOE_OK


def test_binding_raises_without_a_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        L.lib()


def test_kernel_timing_hook_validation():
    lib = M.lib()
    assert lib.moe_set_kernel_events(None, -1) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_set_kernel_events(None, 2) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_set_kernel_events(None, 0) == M.MOE_OK
    # a call rejected by validation launches nothing
    assert _fwd(_bank(), T=-1) == M.MOE_ERR_INVALID_ARG
    assert M.moe_last_call_launches() == 0
    assert M.moe_launch_name(0) is None
    assert M.moe_launch_name(-1) is None


def test_oracle_is_not_imported_by_the_product_path():
    pkg = os.path.dirname(M.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "oracle" not in text.replace("oracle is", ""), f


def test_mxfp8_act_entry_points_validate_before_launching():
    lib = M.lib()
    b = _bank(E=16, H=256, I=128)
    fwd = lambda bank, T=8, k=2, x=FAKE, ws_bytes=1 << 40: lib.moe_layer_forward_mxfp8_act(
        x, FAKE, None, ctypes.byref(bank), None, T, k, FAKE, None, None, FAKE, ws_bytes, None)
    assert fwd(b, x=None) == M.MOE_ERR_INVALID_ARG
    assert fwd(_bank(E=16, H=160, I=128)) == M.MOE_ERR_UNSUPPORTED   # H not a multiple of 256
    assert fwd(_bank(E=16, H=256, I=96)) == M.MOE_ERR_UNSUPPORTED    # I not a multiple of 128
    assert fwd(b, ws_bytes=16) == M.MOE_ERR_WORKSPACE
    assert fwd(b, T=0) == M.MOE_OK
    q = lib.moe_quantize_mxfp8
    assert q(FAKE, 4, 48, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG      # H % 32
    assert q(FAKE, -1, 64, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert q(FAKE + 2, 4, 64, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG  # misaligned x
    assert q(None, 4, 64, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert q(None, 0, 64, None, None, None) == M.MOE_OK
    # the workspace covers the mode at every size
    for T in (1, 300, 16384):
        assert M.moe_workspace_bytes(T, 5120, 2304, 384, 6) >= T * 5120 * 33 // 32


def test_fp8_entry_points_validate_before_launching():
    lib = M.lib()
    good = L.Fp8Bank(FAKE, FAKE, FAKE, FAKE, 1, 256, 128)
    ffn = lambda b, T=4, ws_bytes=1 << 40, x=FAKE: lib.moe_expert_ffn_fp8(
        x, ctypes.byref(b), T, FAKE, FAKE, ws_bytes, None)
    assert ffn(good, x=None) == M.MOE_ERR_INVALID_ARG
    assert ffn(L.Fp8Bank(FAKE, FAKE, FAKE, FAKE, 2, 256, 128)) == M.MOE_ERR_INVALID_ARG   # E != 1
    assert ffn(L.Fp8Bank(FAKE + 4, FAKE, FAKE, FAKE, 1, 256, 128)) == M.MOE_ERR_INVALID_ARG
    assert ffn(L.Fp8Bank(FAKE, FAKE, FAKE, FAKE, 1, 250, 128)) == M.MOE_ERR_INVALID_ARG   # H % 32
    assert ffn(good, ws_bytes=16) == M.MOE_ERR_WORKSPACE
    assert ffn(good, T=0) == M.MOE_OK
    routed = _bank(E=16, H=256, I=128)
    fwd = lambda sh, T=8: lib.moe_layer_forward_fp8_shared(
        FAKE, FAKE, None, ctypes.byref(routed), None if sh is None else ctypes.byref(sh), T, 2,
        FAKE, None, None, FAKE, 1 << 40, None)
    assert fwd(None) == M.MOE_ERR_INVALID_ARG
    assert fwd(L.Fp8Bank(FAKE, FAKE, FAKE, FAKE, 1, 256, 96)) == M.MOE_ERR_INVALID_ARG   # I mismatch
    assert fwd(good, T=0) == M.MOE_OK
    # the workspace size covers the FP8 paths at every size
    for T in (1, 5, 16, 17, 2048):
        assert M.moe_workspace_bytes(T, 5120, 2304, 384, 6) >= T * 5120 * 4


def test_nvfp4_entry_points_validate_before_launching():
    lib = M.lib()
    good = L.NvBank(FAKE, FAKE, FAKE, FAKE, None, 16, 256, 128)
    fwd = lambda b, sh=None, T=8, k=2, ws_bytes=1 << 40: lib.moe_layer_forward_nvfp4(
        FAKE, FAKE, None, ctypes.byref(b), None if sh is None else ctypes.byref(sh), T, k, FAKE,
        None, None, FAKE, ws_bytes, None)
    assert fwd(L.NvBank(FAKE, FAKE + 2, FAKE, FAKE, None, 16, 256, 128)) == M.MOE_ERR_INVALID_ARG
    assert fwd(L.NvBank(FAKE + 4, FAKE, FAKE, FAKE, None, 16, 256, 128)) == M.MOE_ERR_INVALID_ARG
    assert fwd(good, sh=L.NvBank(FAKE, FAKE, FAKE, FAKE, None, 2, 256, 128)) == M.MOE_ERR_INVALID_ARG
    assert fwd(good, k=17) == M.MOE_ERR_INVALID_ARG
    assert fwd(good, ws_bytes=16) == M.MOE_ERR_WORKSPACE
    assert fwd(good, T=0) == M.MOE_OK
    ffn = lambda b, R=8, off=FAKE: lib.moe_expert_ffn_nvfp4(FAKE, ctypes.byref(b), off, FAKE, 8, R,
                                                           FAKE, FAKE, 1 << 40, None)
    assert ffn(good, off=None) == M.MOE_ERR_INVALID_ARG   # E > 1 needs offsets
    assert ffn(good, R=-1) == M.MOE_ERR_INVALID_ARG
    assert ffn(good, R=0) == M.MOE_OK


def test_workspace_status_rejects_a_null_workspace_without_a_device_call():
    assert M.lib().moe_workspace_status(None) == M.MOE_ERR_INVALID_ARG
    assert M.lib().moe_set_wait_test(0) == M.MOE_OK
