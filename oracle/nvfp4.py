"""fp64 oracle of the layer with its experts in NVFP4.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and bench.py's CPU-baseline leg use it; the HIP library never does.

The pages name NVFP4 as a format other engines load V4.1's experts in
(FreeToken issue #444, the comment listing what another pull request covers:
"NVFP4 experts"; the same issue, "Is the quantization already supported":
FP8 and NVFP4 among the formats the engine supports; ai.rs article, its
reading list)
and describe its element-and-scale layout where they describe the model's
fp4 KV cache: E2M1 elements with one E4M3 scale per 16 (FreeToken issue #444,
"Architecture delta vs deepseek_v4", its list of what is new).

Readings (the pages give no more than that):
* codes are packed exactly like the MXFP4 banks (byte b of a row holds
  elements 2b, 2b+1 in its low and high nibble; E2M1 as in OCP MX);
* one E4M3 scale byte (OCP fp8, positive in practice; its sign is honoured)
  per 16 consecutive elements along K: scales [N][K/16];
* one fp32 scale per (expert, matrix): global_scales [E][3] (gate, up, down)
  multiplies the whole matrix; absent means 1;
* an NVFP4 bank: gate_up_codes [E][2][I][H/2], gate_up_scales [E][2][I][H/16],
  down_codes [E][H][I/2], down_scales [E][H][I/16], global_scales [E][3].
Routing, SwiGLU, the shared expert and the combine are those of oracle.moe.
"""

from __future__ import annotations

import numpy as np

from . import moe as O
from .mxfp8_act import e4m3_to_f64


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, global_scale: float = 1.0) -> np.ndarray:
    """Packed E2M1 codes [N][K/2] + E4M3 scales [N][K/16] (+ fp32 matrix scale)
    -> fp64 [N][K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, half = codes.shape
    K = 2 * half
    if scales.shape != (N, K // 16):
        raise ValueError("scales must be [N][K/16]")
    idx = np.empty((N, K), dtype=np.uint8)
    idx[:, 0::2] = codes & 0x0F
    idx[:, 1::2] = codes >> 4
    w = O.E2M1_TABLE[idx].reshape(N, K // 16, 16) * e4m3_to_f64(scales)[:, :, None]
    return w.reshape(N, K) * float(global_scale)


def expert_weights_nvfp4(bank: dict, e: int):
    g = bank.get("global_scales")
    gs = (1.0, 1.0, 1.0) if g is None else tuple(float(v) for v in np.asarray(g, np.float32)[e])
    wg = dequant_nvfp4(bank["gate_up_codes"][e, 0], bank["gate_up_scales"][e, 0], gs[0])
    wu = dequant_nvfp4(bank["gate_up_codes"][e, 1], bank["gate_up_scales"][e, 1], gs[1])
    wd = dequant_nvfp4(bank["down_codes"][e], bank["down_scales"][e], gs[2])
    return wg, wu, wd


def expert_bytes_nvfp4(H: int, I: int) -> int:
    """1/2 byte per code, 1 byte per 16 codes, 12 bytes of matrix scales."""
    n = 3 * H * I
    return n // 2 + n // 16 + 12


def expert_rows_nvfp4(x: np.ndarray, bank: dict, offsets, row_token, rows=None) -> np.ndarray:
    R = len(row_token)
    y = np.full((R, x.shape[1]), np.nan)
    want = np.ones(R, bool) if rows is None else np.isin(np.arange(R), rows)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sel = [r for r in range(lo, hi) if want[r]]
        if sel:
            y[sel] = O.expert_ffn(x[row_token[sel]], *expert_weights_nvfp4(bank, e))
    return y


def layer_nvfp4(x_bits, w_router_bits, bias, routed: dict, shared: dict | None, k: int,
                tokens=None) -> dict:
    """The layer with NVFP4 routed (and shared) experts, in fp64."""
    r = O.route(x_bits, w_router_bits, bias, k)
    x = r["x"]
    T = x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    rows = r["inv_row"][tok].reshape(-1)
    y_rows = expert_rows_nvfp4(x, routed, r["offsets"], r["row_token"],
                               None if tokens is None else rows)
    y_sh = None if shared is None else O.expert_ffn(x[tok], *expert_weights_nvfp4(shared, 0))
    out = O.combine(y_rows, r["inv_row"][tok], r["w"][tok], y_sh)
    r.update(y_rows=y_rows, y_shared=y_sh, out=out, tokens=tok)
    return r


def token_out_with_nvfp4(x: np.ndarray, L: np.ndarray, t: int, ids, routed: dict,
                         y_shared_t=None) -> np.ndarray:
    ids = np.asarray(ids)
    w = O.topk_weights(L[t:t + 1], ids[None, :])[0]
    out = np.zeros(x.shape[1]) if y_shared_t is None else y_shared_t.copy()
    for j, e in enumerate(ids):
        out = out + w[j] * O.expert_ffn(x[t:t + 1], *expert_weights_nvfp4(routed, int(e)))[0]
    return out
