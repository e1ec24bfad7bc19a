"""fp64 oracle of an FP8 expert with 32 x 32 block scales (the checkpoint's
dense format) and of the layer whose shared expert is stored that way.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and bench.py's CPU-baseline leg use it; the HIP library never does.

The pages: the reference checkpoint stores its dense weights in fp8 with
32 x 32 weight blocks and ue8m0 scales, and its routed experts in fp4
(FreeToken issue #444, "Is the quantization already supported"); moving
from 128 x 128 to 32 x 32 scale blocks is one of the silent
incompatibilities they warn about, since every shape stays valid while each
dequantised weight comes out mis-scaled (ai.rs article on
DeepSeek-V4.1-Flash, "The defect that never raised an error"; FreeToken
issue #444, angelbaba01L's comment pointing at the port's write-up). The shared expert gets the same input and
arithmetic as the routed ones (ai.rs article on DeepSeek-V4.1-Flash, "What
remains is the reference rounding itself").

Readings (the pages give the block size and scale format only):
* elements are OCP E4M3 bytes (the fp8 format of MX and of gfx950);
* block (i, j) covers rows 32i..32i+31 and columns 32j..32j+31 of a matrix
  stored [N][K] (rows = outputs, K = the reduction dimension, not
  transposed, like the fp4 banks); its scale byte s multiplies the block by
  2^(s - 127), s == 255 is NaN;
* an FP8 bank: gate_up [E][2][I][H] with scales [E][2][I/32][H/32], down
  [E][H][I] with scales [E][H/32][I/32]; the shared expert is E = 1.

Everything is fp64 from the bit-level inputs.
"""

from __future__ import annotations

import numpy as np

from . import moe as O
from .mxfp8_act import e4m3_to_f64


def dequant_fp8_block32(w: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 bytes [N][K] + E8M0 scales [N/32][K/32] -> fp64 [N][K]."""
    w = np.asarray(w, dtype=np.uint8)
    N, K = w.shape
    if scales.shape != (N // 32, K // 32):
        raise ValueError("scales must be [N/32][K/32]")
    v = e4m3_to_f64(w).reshape(N // 32, 32, K // 32, 32)
    v = v * O.e8m0_to_f64(scales)[:, None, :, None]
    return v.reshape(N, K)


def expert_weights_fp8(bank: dict, e: int):
    """(W_gate [I][H], W_up [I][H], W_down [H][I]) of expert e, fp64."""
    wg = dequant_fp8_block32(bank["gate_up_w"][e, 0], bank["gate_up_scales"][e, 0])
    wu = dequant_fp8_block32(bank["gate_up_w"][e, 1], bank["gate_up_scales"][e, 1])
    wd = dequant_fp8_block32(bank["down_w"][e], bank["down_scales"][e])
    return wg, wu, wd


def expert_bytes_fp8(H: int, I: int) -> int:
    """One byte per weight plus one scale byte per 32 x 32 block."""
    n = 3 * H * I
    return n + n // 1024


def dense_ffn_fp8(x: np.ndarray, bank: dict, e: int = 0) -> np.ndarray:
    """SwiGLU of every row of x [T][H] through FP8 expert e."""
    return O.expert_ffn(x, *expert_weights_fp8(bank, e))


def layer_fp8_shared(x_bits, w_router_bits, bias, routed: dict, shared_fp8: dict, k: int,
                     tokens=None) -> dict:
    """The layer with MXFP4 routed experts and an FP8 shared expert: routing,
    routed rows and combine as in oracle.moe.layer; the shared row from the
    FP8 weights."""
    r = O.route(x_bits, w_router_bits, bias, k)
    x = r["x"]
    T = x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    rows = r["inv_row"][tok].reshape(-1)
    y_rows = O.expert_rows(x, routed, r["offsets"], r["row_token"],
                           None if tokens is None else rows)
    y_sh = dense_ffn_fp8(x[tok], shared_fp8)
    out = O.combine(y_rows, r["inv_row"][tok], r["w"][tok], y_sh)
    r.update(y_rows=y_rows, y_shared=y_sh, out=out, tokens=tok)
    return r
