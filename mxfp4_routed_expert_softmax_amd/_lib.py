"""ctypes binding of libmoe_mxfp4.so (the C ABI in include/moe_mxfp4.h).

Argument marshalling only: torch device tensors become device pointers and
the current HIP stream becomes the stream argument; every step of the layer
runs in the library's kernels. There is no fallback: if the library is not
built, or its call fails, these functions raise.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_MXFP4_LIB points the binding at another build of the same library
LIB_PATH = os.environ.get("MOE_MXFP4_LIB") or os.path.join(PKG, "libmoe_mxfp4.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe_mxfp4.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_TIMEOUT = -5


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {status} ({msg})")
        self.status = status


class Bank(ctypes.Structure):
    """moe_mxfp4_bank: device pointers of one MXFP4 bank plus its sizes."""

    _fields_ = [
        ("gate_up_codes", ctypes.c_void_p),
        ("gate_up_scales", ctypes.c_void_p),
        ("down_codes", ctypes.c_void_p),
        ("down_scales", ctypes.c_void_p),
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
    ]


class Fp8Bank(ctypes.Structure):
    """moe_fp8_bank: device pointers of one FP8 (32 x 32 block-scaled) bank."""

    _fields_ = [
        ("gate_up_w", ctypes.c_void_p),
        ("gate_up_scales", ctypes.c_void_p),
        ("down_w", ctypes.c_void_p),
        ("down_scales", ctypes.c_void_p),
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
    ]


class NvBank(ctypes.Structure):
    """moe_nvfp4_bank: device pointers of one NVFP4 bank plus its sizes."""

    _fields_ = [
        ("gate_up_codes", ctypes.c_void_p),
        ("gate_up_scales", ctypes.c_void_p),
        ("down_codes", ctypes.c_void_p),
        ("down_scales", ctypes.c_void_p),
        ("global_scales", ctypes.c_void_p),
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "moe_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_router_topk": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn_mxfp4": (_I, [_P, ctypes.POINTER(Bank), _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "moe_combine": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_layer_forward": (_I, [_P, _P, _P, ctypes.POINTER(Bank), ctypes.POINTER(Bank), _I, _I,
                                _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_mxfp8_act": (_I, [_P, _P, _P, ctypes.POINTER(Bank), ctypes.POINTER(Bank),
                                          _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_noalloc": (_I, [_P, _P, _P, ctypes.POINTER(Bank), ctypes.POINTER(Bank),
                                        _I, _I, _P, _P, _P, _P]),
    "moe_quantize_mxfp8": (_I, [_P, _I, _I, _P, _P, _P]),
    "moe_expert_ffn_fp8": (_I, [_P, ctypes.POINTER(Fp8Bank), _I, _P, _P, _SZ, _P]),
    "moe_expert_ffn_nvfp4": (_I, [_P, ctypes.POINTER(NvBank), _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "moe_layer_forward_nvfp4": (_I, [_P, _P, _P, ctypes.POINTER(NvBank), ctypes.POINTER(NvBank),
                                      _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_fp8_shared": (_I, [_P, _P, _P, ctypes.POINTER(Bank), ctypes.POINTER(Fp8Bank),
                                           _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_set_kernel_events": (_I, [_P, _I]),
    "moe_last_call_launches": (_I, []),
    "moe_workspace_status": (_I, [_P]),
    "moe_set_wait_test": (_I, [_I]),
    "moe_launch_name": (ctypes.c_char_p, [_I]),
}

_lib = None


def header_functions() -> list[str]:
    """Names of the functions declared in include/moe_mxfp4.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mxfp4_routed_expert_softmax_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status, status_str(status))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream, ref) -> int:
    import torch
    if stream is None:
        dev = ref.device if ref is not None else torch.device("cuda")
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, name, dtypes, ndim=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.uint16, torch.int16)


class BankTensors:
    """Keeps the four bank tensors alive next to their ctypes struct."""

    def __init__(self, gate_up_codes, gate_up_scales, down_codes, down_scales):
        import torch
        for n, t in [("gate_up_codes", gate_up_codes), ("gate_up_scales", gate_up_scales),
                     ("down_codes", down_codes), ("down_scales", down_scales)]:
            _need(t, n, (torch.uint8,))
        E, two, I, h2 = gate_up_codes.shape
        H = 2 * h2
        if two != 2 or tuple(gate_up_scales.shape) != (E, 2, I, H // 32) \
                or tuple(down_codes.shape) != (E, H, I // 2) \
                or tuple(down_scales.shape) != (E, H, I // 32):
            raise ValueError("bank tensors do not have the [E][2][I][H/2] ... layout")
        self.tensors = (gate_up_codes, gate_up_scales, down_codes, down_scales)
        self.E, self.H, self.I = E, H, I
        self.struct = Bank(gate_up_codes.data_ptr(), gate_up_scales.data_ptr(),
                           down_codes.data_ptr(), down_scales.data_ptr(), E, H, I)

    @classmethod
    def from_numpy(cls, arrs: dict, device="cuda"):
        import torch
        t = {k: torch.from_numpy(arrs[k]).to(device) for k in
             ("gate_up_codes", "gate_up_scales", "down_codes", "down_scales")}
        return cls(t["gate_up_codes"], t["gate_up_scales"], t["down_codes"], t["down_scales"])


class Fp8BankTensors:
    """Keeps the four FP8 bank tensors alive next to their ctypes struct."""

    def __init__(self, gate_up_w, gate_up_scales, down_w, down_scales):
        import torch
        for n, t in [("gate_up_w", gate_up_w), ("gate_up_scales", gate_up_scales),
                     ("down_w", down_w), ("down_scales", down_scales)]:
            _need(t, n, (torch.uint8,))
        E, two, I, H = gate_up_w.shape
        if two != 2 or tuple(gate_up_scales.shape) != (E, 2, I // 32, H // 32) \
                or tuple(down_w.shape) != (E, H, I) \
                or tuple(down_scales.shape) != (E, H // 32, I // 32):
            raise ValueError("FP8 bank tensors do not have the [E][2][I][H] ... layout")
        self.tensors = (gate_up_w, gate_up_scales, down_w, down_scales)
        self.E, self.H, self.I = E, H, I
        self.struct = Fp8Bank(gate_up_w.data_ptr(), gate_up_scales.data_ptr(),
                              down_w.data_ptr(), down_scales.data_ptr(), E, H, I)

    @classmethod
    def from_numpy(cls, arrs: dict, device="cuda"):
        import torch
        t = {k: torch.from_numpy(arrs[k]).to(device) for k in
             ("gate_up_w", "gate_up_scales", "down_w", "down_scales")}
        return cls(t["gate_up_w"], t["gate_up_scales"], t["down_w"], t["down_scales"])


class NvBankTensors:
    """Keeps the NVFP4 bank tensors alive next to their ctypes struct."""

    def __init__(self, gate_up_codes, gate_up_scales, down_codes, down_scales,
                 global_scales=None):
        import torch
        for n, t in [("gate_up_codes", gate_up_codes), ("gate_up_scales", gate_up_scales),
                     ("down_codes", down_codes), ("down_scales", down_scales)]:
            _need(t, n, (torch.uint8,))
        E, two, I, h2 = gate_up_codes.shape
        H = 2 * h2
        if two != 2 or tuple(gate_up_scales.shape) != (E, 2, I, H // 16) \
                or tuple(down_codes.shape) != (E, H, I // 2) \
                or tuple(down_scales.shape) != (E, H, I // 16):
            raise ValueError("NVFP4 bank tensors do not have the [E][2][I][H/2] ... layout")
        if global_scales is not None:
            _need(global_scales, "global_scales", (torch.float32,))
            if tuple(global_scales.shape) != (E, 3):
                raise ValueError("global_scales must be [E][3]")
        self.tensors = (gate_up_codes, gate_up_scales, down_codes, down_scales, global_scales)
        self.E, self.H, self.I = E, H, I
        self.struct = NvBank(gate_up_codes.data_ptr(), gate_up_scales.data_ptr(),
                             down_codes.data_ptr(), down_scales.data_ptr(),
                             None if global_scales is None else global_scales.data_ptr(), E, H, I)

    @classmethod
    def from_numpy(cls, arrs: dict, device="cuda"):
        import torch
        t = {k: torch.from_numpy(arrs[k]).to(device) for k in
             ("gate_up_codes", "gate_up_scales", "down_codes", "down_scales")}
        g = arrs.get("global_scales")
        g = None if g is None else torch.from_numpy(np.asarray(g, np.float32)).to(device)
        return cls(t["gate_up_codes"], t["gate_up_scales"], t["down_codes"], t["down_scales"], g)


# ---------------------------------------------------------------------------
# The C ABI, one Python function per entry point
# ---------------------------------------------------------------------------

def moe_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_workspace_bytes(T, H, I, E, k))


def workspace(T: int, H: int, I: int, E: int, k: int, device="cuda"):
    """A uint8 device tensor of moe_workspace_bytes(...) bytes."""
    import torch
    return torch.empty(max(moe_workspace_bytes(T, H, I, E, k), 256), dtype=torch.uint8,
                       device=device)


def moe_router_topk(x, w_router, logit_bias, k, topk_ids, topk_w, logits_out=None, ws=None,
                    stream=None):
    import torch
    _need(x, "x", _bf16_types(), 2)
    _need(w_router, "w_router", _bf16_types(), 2)
    _need(topk_ids, "topk_ids", (torch.int32,))
    _need(topk_w, "topk_w", (torch.float32,))
    if logit_bias is not None:
        _need(logit_bias, "logit_bias", (torch.float32,))
    if logits_out is not None:
        _need(logits_out, "logits_out", (torch.float32,))
    T, H = x.shape
    E = w_router.shape[0]
    st = lib().moe_router_topk(_ptr(x), _ptr(w_router), _ptr(logit_bias), T, H, E, k,
                               _ptr(topk_ids), _ptr(topk_w), _ptr(logits_out), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream, x))
    _check("moe_router_topk", st)


def moe_permute(topk_ids, E, expert_offsets, row_token, inv_row, ws, stream=None):
    import torch
    _need(topk_ids, "topk_ids", (torch.int32,), 2)
    for n, t in [("expert_offsets", expert_offsets), ("row_token", row_token),
                 ("inv_row", inv_row)]:
        _need(t, n, (torch.int32,))
    T, k = topk_ids.shape
    st = lib().moe_permute(_ptr(topk_ids), T, k, E, _ptr(expert_offsets), _ptr(row_token),
                           _ptr(inv_row), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(),
                           _stream(stream, topk_ids))
    _check("moe_permute", st)


def moe_expert_ffn_mxfp4(x, bank: BankTensors, expert_offsets, row_token, R, y_rows, ws,
                         stream=None):
    import torch
    _need(x, "x", _bf16_types(), 2)
    _need(y_rows, "y_rows", (torch.float32,))
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", (torch.int32,))
    if row_token is not None:
        _need(row_token, "row_token", (torch.int32,))
    T = x.shape[0]
    st = lib().moe_expert_ffn_mxfp4(_ptr(x), ctypes.byref(bank.struct), _ptr(expert_offsets),
                                    _ptr(row_token), T, R, _ptr(y_rows), _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream, x))
    _check("moe_expert_ffn_mxfp4", st)


def moe_combine(y_rows, inv_row, topk_w, y_shared, out, stream=None):
    import torch
    _need(inv_row, "inv_row", (torch.int32,), 2)
    _need(topk_w, "topk_w", (torch.float32,), 2)
    _need(out, "out", (torch.float32,), 2)
    if y_rows is not None:
        _need(y_rows, "y_rows", (torch.float32,))
    if y_shared is not None:
        _need(y_shared, "y_shared", (torch.float32,))
    T, k = inv_row.shape
    H = out.shape[1]
    R = 0 if y_rows is None else y_rows.shape[0]
    st = lib().moe_combine(_ptr(y_rows), _ptr(inv_row), _ptr(topk_w), _ptr(y_shared), T, k, H,
                           R, _ptr(out), _stream(stream, out))
    _check("moe_combine", st)


def _layer(fn, x, w_router, logit_bias, routed, shared, k, out, topk_ids_out, topk_w_out, ws,
           stream):
    import torch
    _need(x, "x", _bf16_types(), 2)
    _need(w_router, "w_router", _bf16_types(), 2)
    _need(out, "out", (torch.float32,), 2)
    if logit_bias is not None:
        _need(logit_bias, "logit_bias", (torch.float32,))
    T = x.shape[0]
    st = getattr(lib(), fn)(
        _ptr(x), _ptr(w_router), _ptr(logit_bias), ctypes.byref(routed.struct),
        None if shared is None else ctypes.byref(shared.struct), T, k, _ptr(out),
        _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream, x))
    _check(fn, st)


def moe_layer_forward(x, w_router, logit_bias, routed: BankTensors, shared: BankTensors | None,
                      k, out, topk_ids_out=None, topk_w_out=None, ws=None, stream=None):
    _layer("moe_layer_forward", x, w_router, logit_bias, routed, shared, k, out, topk_ids_out,
           topk_w_out, ws, stream)


def moe_layer_forward_noalloc(x, w_router, logit_bias, routed: BankTensors,
                              shared: BankTensors | None, k, out, topk_ids_out=None,
                              topk_w_out=None, stream=None):
    """moe_layer_forward on the library's own fixed per-GPU scratch (no
    workspace argument; the call allocates nothing)."""
    import torch
    _need(x, "x", _bf16_types(), 2)
    _need(w_router, "w_router", _bf16_types(), 2)
    _need(out, "out", (torch.float32,), 2)
    if logit_bias is not None:
        _need(logit_bias, "logit_bias", (torch.float32,))
    st = lib().moe_layer_forward_noalloc(
        _ptr(x), _ptr(w_router), _ptr(logit_bias), ctypes.byref(routed.struct),
        None if shared is None else ctypes.byref(shared.struct), x.shape[0], k, _ptr(out),
        _ptr(topk_ids_out), _ptr(topk_w_out), _stream(stream, x))
    _check("moe_layer_forward_noalloc", st)


def moe_layer_forward_mxfp8_act(x, w_router, logit_bias, routed: BankTensors,
                                shared: BankTensors | None, k, out, topk_ids_out=None,
                                topk_w_out=None, ws=None, stream=None):
    _layer("moe_layer_forward_mxfp8_act", x, w_router, logit_bias, routed, shared, k, out,
           topk_ids_out, topk_w_out, ws, stream)


def moe_expert_ffn_fp8(x, bank: Fp8BankTensors, y, ws, stream=None):
    import torch
    _need(x, "x", _bf16_types(), 2)
    _need(y, "y", (torch.float32,), 2)
    T = x.shape[0]
    st = lib().moe_expert_ffn_fp8(_ptr(x), ctypes.byref(bank.struct), T, _ptr(y), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream, x))
    _check("moe_expert_ffn_fp8", st)


def moe_layer_forward_fp8_shared(x, w_router, logit_bias, routed: BankTensors,
                                 shared: Fp8BankTensors, k, out, topk_ids_out=None,
                                 topk_w_out=None, ws=None, stream=None):
    _layer("moe_layer_forward_fp8_shared", x, w_router, logit_bias, routed, shared, k, out,
           topk_ids_out, topk_w_out, ws, stream)


def moe_expert_ffn_nvfp4(x, bank: NvBankTensors, expert_offsets, row_token, R, y_rows, ws,
                         stream=None):
    import torch
    _need(x, "x", _bf16_types(), 2)
    _need(y_rows, "y_rows", (torch.float32,))
    T = x.shape[0]
    st = lib().moe_expert_ffn_nvfp4(_ptr(x), ctypes.byref(bank.struct), _ptr(expert_offsets),
                                    _ptr(row_token), T, R, _ptr(y_rows), _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream, x))
    _check("moe_expert_ffn_nvfp4", st)


def moe_layer_forward_nvfp4(x, w_router, logit_bias, routed: NvBankTensors,
                            shared: NvBankTensors | None, k, out, topk_ids_out=None,
                            topk_w_out=None, ws=None, stream=None):
    _layer("moe_layer_forward_nvfp4", x, w_router, logit_bias, routed, shared, k, out,
           topk_ids_out, topk_w_out, ws, stream)


def moe_quantize_mxfp8(x, codes, scales, stream=None):
    import torch
    _need(x, "x", _bf16_types(), 2)
    _need(codes, "codes", (torch.uint8,))
    _need(scales, "scales", (torch.uint8,))
    T, H = x.shape
    if codes.numel() != T * H or scales.numel() != T * (H // 32):
        raise ValueError("codes must hold T*H bytes and scales T*H/32")
    st = lib().moe_quantize_mxfp8(_ptr(x), T, H, _ptr(codes), _ptr(scales), _stream(stream, x))
    _check("moe_quantize_mxfp8", st)


def moe_set_kernel_events(events, n: int) -> None:
    """Timing hook: `events` is a ctypes array of n hipEvent_t handles (or
    None with n = 0 to turn the hook off)."""
    _check("moe_set_kernel_events", lib().moe_set_kernel_events(events, n))


def moe_last_call_launches() -> int:
    return int(lib().moe_last_call_launches())


def moe_launch_name(i: int) -> str | None:
    r = lib().moe_launch_name(i)
    return None if r is None else r.decode()


def moe_workspace_status(ws) -> int:
    """Wait status of the last few-token call made with workspace `ws`
    (MOE_OK or MOE_ERR_TIMEOUT); a blocking 16-byte copy, so synchronise
    the call's stream first. Raises on other errors."""
    st = lib().moe_workspace_status(_ptr(ws))
    if st not in (MOE_OK, MOE_ERR_TIMEOUT):
        _check("moe_workspace_status", st)
    return st


def moe_set_wait_test(on: bool) -> None:
    """Test hook: while on, the routing's first bounded wait of every
    few-token layer call from this thread gives up after a few polls."""
    _check("moe_set_wait_test", lib().moe_set_wait_test(1 if on else 0))
