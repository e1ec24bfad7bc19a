"""fp64 oracle of the layer with MXFP8 activations (the opt-in native-MX mode).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and bench.py's CPU-baseline leg use it; the HIP library never does.

The mode: the expert FFNs take their activations rounded to MXFP8 (E4M3
elements with one E8M0 scale per 32 along the reduction dimension), so that
both operands of every expert product are microscaled and the matrix cores
can take the MXFP4 weight codes as they are. The pages describe the
reference model running its linear layers in fp8 with block scales and
dynamically rounded activations (FreeToken issue #444, "Is the quantization
already supported": the checkpoint's quantisation config with a dynamic
activation scheme and ue8m0 scales; ai.rs article on DeepSeek-V4.1-Flash, "What remains
is the reference rounding itself", which also tabulates what one fp8 linear
layer's rounding costs against full precision). Which activations are
rounded, and how, the pages leave open; the readings taken here:

* the router keeps the exact bf16 activations (its top-k is a discrete
  switch, the most error-sensitive step the pages name);
* x is rounded once per token row (blocks of 32 along H) and feeds the
  gate/up products of every expert of the token, routed and shared;
* h = silu(g) * u is rounded per row (blocks of 32 along I) before the down
  product;
* the rounding is the OCP Microscaling v1.0 conversion: block scale
  2^(floor(log2(amax)) - 8) (8 = the largest E4M3 exponent), clamped to the
  E8M0 range; each element divided by it and rounded to nearest-even E4M3,
  magnitudes beyond the largest normal (448) clamped to it; an all-zero block
  takes scale byte 0. The sign of every element is kept (negative values
  that round to zero give the -0 code 0x80).

Everything is fp64; the expert weights are the exact MXFP4 dequantisation of
oracle.moe.
"""

from __future__ import annotations

import numpy as np

from . import moe as O

E4M3_MAX = 448.0
E4M3_EMAX = 8


def e4m3_to_f64(b: np.ndarray) -> np.ndarray:
    """E4M3 byte (OCP FP8: 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 subnormal m/8 * 2^-6; S.1111.111 NaN, no infinities)
    -> fp64."""
    b = np.asarray(b).astype(np.int64)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(b & 0x80, -mag, mag)


def _round_e4m3(q: np.ndarray) -> np.ndarray:
    """Magnitudes q >= 0 (already divided by the block scale) -> E4M3
    magnitude codes 0..0x7E, nearest with ties to even, clamped to 448."""
    q = np.asarray(q, dtype=np.float64)
    code = np.zeros(q.shape, dtype=np.int64)
    sub = q < 2.0 ** -6
    # subnormal range: steps of 2^-9; a count of 8 steps is the code of 2^-6
    code[sub] = np.rint(q[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if nrm.any():
        qn = q[nrm]
        e = np.floor(np.log2(qn)).astype(np.int64)
        # guard log2 rounding at exact powers of two
        e = np.where(np.ldexp(1.0, e) > qn, e - 1, e)
        e = np.where(np.ldexp(1.0, e + 1) <= qn, e + 1, e)
        e = np.minimum(e, E4M3_EMAX)
        steps = np.rint(qn / np.ldexp(1.0, e - 3)).astype(np.int64)  # 8..16 (or more when clamped)
        # a carry to 16 steps moves to the next binade: value = steps * 2^(e-3)
        c = ((e + 7) << 3) + (steps - 8)
        code[nrm] = np.minimum(c, 0x7E)
    return code


def quantise_mxfp8(v: np.ndarray):
    """fp64 [..., K] (K a multiple of 32) -> (codes uint8 [..., K],
    scales uint8 [..., K/32]): one E8M0 scale per 32 consecutive values."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.max(np.abs(blk), axis=-1)
    with np.errstate(divide="ignore"):
        se = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64)
    pos = amax > 0
    se = np.where(pos & (np.ldexp(1.0, se) > amax), se - 1, se)
    se = np.where(pos & (np.ldexp(1.0, se + 1) <= amax), se + 1, se)
    se = np.clip(se - E4M3_EMAX, -127, 127)
    se = np.where(pos, se, -127)
    q = np.abs(blk) / np.ldexp(1.0, se)[..., None]
    mag = _round_e4m3(q)
    codes = (mag | np.where(np.signbit(blk), 0x80, 0)).astype(np.uint8)
    scales = (se + 127).astype(np.uint8)
    return codes.reshape(v.shape), scales


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [..., K] + E8M0 scales [..., K/32] -> fp64 [..., K]."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    v = e4m3_to_f64(codes).reshape(codes.shape[:-1] + (K // 32, 32))
    v = v * O.e8m0_to_f64(scales)[..., None]
    return v.reshape(codes.shape)


def round_mxfp8(v: np.ndarray) -> np.ndarray:
    """The fp64 value each element takes after MXFP8 rounding."""
    return dequant_mxfp8(*quantise_mxfp8(v))


def expert_ffn_mx(Xq: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """SwiGLU expert on rows already rounded to MXFP8; h is rounded to MXFP8
    before the down product."""
    g = Xq @ wg.T
    u = Xq @ wu.T
    return round_mxfp8(O.silu(g) * u) @ wd.T


def expert_rows_mx(xq: np.ndarray, bank: dict, offsets, row_token, rows=None) -> np.ndarray:
    R = len(row_token)
    y = np.full((R, xq.shape[1]), np.nan)
    want = np.ones(R, bool) if rows is None else np.isin(np.arange(R), rows)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sel = [r for r in range(lo, hi) if want[r]]
        if not sel:
            continue
        wg, wu, wd = O.expert_weights(bank, e)
        y[sel] = expert_ffn_mx(xq[row_token[sel]], wg, wu, wd)
    return y


def layer_mx(x_bits, w_router_bits, bias, routed: dict, shared: dict | None, k: int,
             tokens=None) -> dict:
    """The layer with MXFP8 expert activations: routing exactly as in
    oracle.moe.layer (exact bf16 x), expert FFNs on the rounded x."""
    r = O.route(x_bits, w_router_bits, bias, k)
    xq = round_mxfp8(r["x"])
    T = xq.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    rows = r["inv_row"][tok].reshape(-1)
    y_rows = expert_rows_mx(xq, routed, r["offsets"], r["row_token"],
                            None if tokens is None else rows)
    y_sh = None
    if shared is not None:
        wg, wu, wd = O.expert_weights(shared, 0)
        y_sh = expert_ffn_mx(xq[tok], wg, wu, wd)
    out = O.combine(y_rows, r["inv_row"][tok], r["w"][tok], y_sh)
    r.update(xq=xq, y_rows=y_rows, y_shared=y_sh, out=out, tokens=tok)
    return r


def token_out_with_mx(xq: np.ndarray, L: np.ndarray, t: int, ids, routed: dict,
                      y_shared_t=None) -> np.ndarray:
    """out[t] of the MX mode for one token with the expert set `ids` (near-tie
    tokens, as oracle.moe.token_out_with)."""
    ids = np.asarray(ids)
    w = O.topk_weights(L[t:t + 1], ids[None, :])[0]
    out = np.zeros(xq.shape[1]) if y_shared_t is None else y_shared_t.copy()
    for j, e in enumerate(ids):
        wg, wu, wd = O.expert_weights(routed, int(e))
        out = out + w[j] * expert_ffn_mx(xq[t:t + 1], wg, wu, wd)[0]
    return out
