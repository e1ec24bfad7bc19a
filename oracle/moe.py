"""fp64 CPU oracle of the routed MXFP4 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the tests, the smoke check of the graft entry point and the
CPU-baseline leg of bench.py do. It shares no code, table or helper with the
HIP library; it reads only the seeded byte/bit arrays both sides consume.

What the layer computes, and where the pages speak of it:

* 384 routed experts per layer, 6 chosen per token, plus 1 shared expert
  (ai.rs article on DeepSeek-V4.1-Flash, table in "What V4.1 Flash is, in
  bytes"; FreeToken issue #444, "Architecture delta vs deepseek_v4").
* Each expert is three 5120 x 2304 FP4 matrices (FreeToken issue #444,
  "Architecture delta vs deepseek_v4"), stored as packed E2M1 codes with one
  E8M0 scale per 32 weights (same issue, janit's comment, section 2 "Routed
  expert bytes per token").
* The shared expert sees the same input and runs the same arithmetic as the
  routed ones (ai.rs article, "What remains is the reference rounding
  itself").
* The routing is a discrete choice whose 6th-to-7th margin is about 1 % of the
  score (same section; llama.cpp discussion #28766, "Correctness"); outputs
  are summed in a fixed order because accumulation order changes results
  (ai.rs article, same section).

Where the pages are silent, this oracle takes these readings (each is listed
with its reason in the design notes): softmax over all E logits, top-k by
descending logit with exact ties to the lower expert id, weights renormalised
over the chosen k (routed scaling 1), SwiGLU y = W_d (silu(W_g x) * (W_u x)),
shared expert added with weight 1, E2M1 values and E8M0 scales as in the OCP
Microscaling v1.0 format (E8M0 byte 255 is NaN), low nibble = even element.

Every value is computed in fp64 from the exact bit-level inputs. The only
library primitives are numpy's fp64 matmul and exp.
"""

from __future__ import annotations

import math
from itertools import combinations

import numpy as np

# ---------------------------------------------------------------------------
# Formats
# ---------------------------------------------------------------------------

# E2M1 (OCP MX v1.0): code = s e1 e0 m. Codes 0-7 are +{0, .5, 1, 1.5, 2, 3,
# 4, 6}; codes 8-15 are the same magnitudes negated (8 is -0).
E2M1_TABLE = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
    dtype=np.float64,
)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e8m0_to_f64(s: np.ndarray) -> np.ndarray:
    """E8M0 scale byte s -> 2**(s - 127); s == 255 encodes NaN."""
    s = np.asarray(s)
    v = np.ldexp(1.0, s.astype(np.int64) - 127)
    return np.where(s == 255, np.nan, v)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed E2M1 codes [N][K/2] + E8M0 scales [N][K/32] -> fp64 [N][K].

    Byte b of a row holds element 2b in its low nibble and 2b+1 in its high
    nibble; scale j multiplies elements 32j .. 32j+31 of the row."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, half = codes.shape
    K = 2 * half
    if scales.shape != (N, K // 32):
        raise ValueError("scales must be [N][K/32]")
    idx = np.empty((N, K), dtype=np.uint8)
    idx[:, 0::2] = codes & 0x0F
    idx[:, 1::2] = codes >> 4
    w = E2M1_TABLE[idx].reshape(N, K // 32, 32)
    w = w * e8m0_to_f64(scales)[:, :, None]
    return w.reshape(N, K)


def expert_weights(bank: dict, e: int):
    """(W_gate [I][H], W_up [I][H], W_down [H][I]) of expert slot e, fp64."""
    wg = dequant_mxfp4(bank["gate_up_codes"][e, 0], bank["gate_up_scales"][e, 0])
    wu = dequant_mxfp4(bank["gate_up_codes"][e, 1], bank["gate_up_scales"][e, 1])
    wd = dequant_mxfp4(bank["down_codes"][e], bank["down_scales"][e])
    return wg, wu, wd


def expert_bytes(H: int, I: int) -> int:
    """Bytes of one MXFP4 expert: three H x I matrices at 1/2 B per code plus
    1 B per 32 codes (FreeToken issue #444, janit's comment, section 2)."""
    n = 3 * H * I
    return n // 2 + n // 32


# ---------------------------------------------------------------------------
# Router: logits, selection, weights
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """L[t][e] = sum_h x[t][h] W_r[e][h] (+ bias[e]); fp64 [T][E]."""
    L = x @ w_router.T
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


def rank_experts(L: np.ndarray) -> np.ndarray:
    """Expert ids of each token ordered by descending logit; exact ties go to
    the lower id (a stable sort of -L keeps ids ascending among equals)."""
    return np.argsort(-L, axis=1, kind="stable")


def select_topk(L: np.ndarray, k: int):
    """ids [T][k] in descending-logit order and the relative margin [T].

    The margin is (p_k - p_{k+1}) / p_k on the softmax probabilities, which
    equals 1 - exp(L_(k+1) - L_(k)); it is +inf when k == E."""
    order = rank_experts(L)
    ids = order[:, :k]
    T, E = L.shape
    if k < E:
        lk = np.take_along_axis(L, order[:, k - 1:k], axis=1)[:, 0]
        lk1 = np.take_along_axis(L, order[:, k:k + 1], axis=1)[:, 0]
        margin = 1.0 - np.exp(lk1 - lk)
    else:
        margin = np.full(T, np.inf)
    return ids, margin


def topk_weights(L: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Routing weights of the chosen experts: the full softmax renormalised
    over the chosen set, written as a softmax over the chosen logits (the
    full-softmax normaliser cancels)."""
    sel = np.take_along_axis(L, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def near_tie_candidates(L_row: np.ndarray, k: int, tol: float = 1.0001e-4,
                        limit: int = 64):
    """All k-subsets S of experts with min(L[S]) >= max(L[not S]) - tol.

    These are the selections that differ from the exact one only by logit
    perturbations below `tol`. Returned as sorted id tuples, the exact
    selection first. Raises if more than `limit` candidates exist."""
    order = rank_experts(L_row[None, :])[0]
    E = L_row.shape[0]
    exact = tuple(sorted(order[:k].tolist()))
    if k == E:
        return [exact]
    lk, lk1 = L_row[order[k - 1]], L_row[order[k]]
    must = [e for e in range(E) if L_row[e] > lk + tol]
    border = [e for e in range(E) if e not in must and L_row[e] >= lk1 - tol]
    need = k - len(must)
    out = [exact]
    n_sub = math.comb(len(border), need) if need >= 0 else 0
    if n_sub > 4 * limit:
        raise ValueError("too many near-tie candidates")
    for sub in combinations(border, need):
        S = tuple(sorted(must + list(sub)))
        if S == exact:
            continue
        inside = L_row[list(S)].min()
        mask = np.ones(E, bool)
        mask[list(S)] = False
        if inside >= L_row[mask].max() - tol:
            out.append(S)
    if len(out) > limit:
        raise ValueError("too many near-tie candidates")
    return out


# ---------------------------------------------------------------------------
# Bucketing
# ---------------------------------------------------------------------------

def permute(ids: np.ndarray, E: int):
    """Stable counting sort of the (token, slot) pairs by expert id.

    Rows are ordered by (expert, token). Returns expert_offsets [E+1],
    row_token [T*k] and inv_row [T][k] (the row holding pair (t, j)).
    The pairs are taken in (t, j) order and sorted by expert with a stable
    sort (a library primitive); a token picks an expert at most once, so the
    order inside a bucket is the token order."""
    T, k = ids.shape
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_token = order // k
    inv = np.empty(T * k, dtype=np.int64)
    inv[order] = np.arange(T * k)
    return offsets, row_token.astype(np.int64), inv.reshape(T, k)


def permute_loops(ids: np.ndarray, E: int):
    """The same bucketing written as plain loops (small inputs only): walk the
    experts in order and, for each, the tokens in order, appending a row for
    every pair that chose it."""
    T, k = ids.shape
    offsets = [0]
    row_token = []
    inv_row = np.full((T, k), -1, dtype=np.int64)
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    inv_row[t, j] = len(row_token)
                    row_token.append(t)
        offsets.append(len(row_token))
    return (np.array(offsets, dtype=np.int64),
            np.array(row_token, dtype=np.int64), inv_row)


# ---------------------------------------------------------------------------
# Expert FFN and combine
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)), fp64 (exp overflow gives -0, as it should)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """SwiGLU expert: rows of X [M][H] -> W_d (silu(W_g x) * (W_u x)), [M][H]."""
    g = X @ wg.T
    u = X @ wu.T
    return (silu(g) * u) @ wd.T


def combine(y_rows: np.ndarray, inv_row: np.ndarray, w: np.ndarray, y_shared=None) -> np.ndarray:
    """out[t] = y_shared[t] + sum_j w[t][j] y_rows[inv_row[t][j]], j = 0..k-1."""
    T, k = inv_row.shape
    out = np.zeros((T, y_rows.shape[1])) if y_shared is None else y_shared.copy()
    for j in range(k):
        out = out + w[:, j:j + 1] * y_rows[inv_row[:, j]]
    return out


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def route(x_bits, w_router_bits, bias, k: int) -> dict:
    """Router half of the layer on every token: logits, ids, weights,
    margins and the bucketing."""
    x = bf16_to_f64(x_bits)
    L = router_logits(x, bf16_to_f64(w_router_bits), bias)
    ids, margin = select_topk(L, k)
    w = topk_weights(L, ids)
    offsets, row_token, inv_row = permute(ids, L.shape[1])
    return dict(x=x, logits=L, ids=ids, w=w, margin=margin,
                offsets=offsets, row_token=row_token, inv_row=inv_row)


def expert_rows(x: np.ndarray, bank: dict, offsets: np.ndarray, row_token: np.ndarray,
                rows=None) -> np.ndarray:
    """y_rows [R][H] of the bucketed rows: row r of bucket e is expert e applied
    to token row_token[r]. `rows` limits the work to a subset (others NaN)."""
    R = len(row_token)
    H = x.shape[1]
    y = np.full((R, H), np.nan)
    want = np.ones(R, bool) if rows is None else np.isin(np.arange(R), rows)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sel = [r for r in range(lo, hi) if want[r]]
        if not sel:
            continue
        wg, wu, wd = expert_weights(bank, e)
        y[sel] = expert_ffn(x[row_token[sel]], wg, wu, wd)
    return y


def shared_out(x: np.ndarray, shared: dict | None, tokens=None) -> np.ndarray | None:
    if shared is None:
        return None
    tokens = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    wg, wu, wd = expert_weights(shared, 0)
    return expert_ffn(x[tokens], wg, wu, wd)


def layer(x_bits, w_router_bits, bias, routed: dict, shared: dict | None, k: int,
          tokens=None) -> dict:
    """The whole layer in fp64.

    With `tokens` given, routing and bucketing cover every token but expert
    outputs and `out` only the listed tokens (out rows in that order)."""
    r = route(x_bits, w_router_bits, bias, k)
    x = r["x"]
    T = x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    rows = r["inv_row"][tok].reshape(-1)
    y_rows = expert_rows(x, routed, r["offsets"], r["row_token"], None if tokens is None else rows)
    y_sh = shared_out(x, shared, tok)
    inv = r["inv_row"][tok]
    out = combine(y_rows, inv, r["w"][tok], y_sh)
    r.update(y_rows=y_rows, y_shared=y_sh, out=out, tokens=tok)
    return r


def token_out_with(x: np.ndarray, L: np.ndarray, t: int, ids, routed: dict,
                   y_shared_t=None) -> np.ndarray:
    """out[t] for one token with the expert set `ids` (weights renormalised
    over that set from the oracle's own logits). Used for near-tie tokens,
    whose valid selections the oracle enumerates itself."""
    ids = np.asarray(ids)
    w = topk_weights(L[t:t + 1], ids[None, :])[0]
    out = np.zeros(x.shape[1]) if y_shared_t is None else y_shared_t.copy()
    for j, e in enumerate(ids):
        wg, wu, wd = expert_weights(routed, int(e))
        out = out + w[j] * expert_ffn(x[t:t + 1], wg, wu, wd)[0]
    return out
