"""Pins of the oracle's near-tie checkers: oracle.moe.token_out_with,
oracle.mxfp8_act.token_out_with_mx and oracle.nvfp4.token_out_with_nvfp4.

These functions give one token's output for an expert set the test names
(the GPU's choice on a token whose k-th and (k+1)-th logits are closer than
the margin), with the routing weights renormalised over that set. Each is
tied here to two things other than itself:

* with the exact selection it must reproduce the whole-layer oracle's row
  (a check of consistency with the pinned layer, for every token);
* with a FORCED, non-exact selection (the 2nd..(k+1)-th ranked experts, and
  a set drawn at random) it must equal a pure-Python evaluation written
  from the definitions: logits by math.fsum over decoded bf16 values, the
  weights exp(L_e - L_max) / sum over the forced set, each expert decoded
  element by element from its bit fields, SwiGLU by fsum dot products, and
  the sum taken in the set's order after the shared row.

A plausible mistake (weights from the exact set instead of the forced one,
an unrenormalised softmax, a dropped or doubled shared row, a wrong expert
index, the wrong rounding point of the MX mode) fails the forced case.
"""

import math

import numpy as np

import synthetic as S
from oracle import moe as O
from oracle import mxfp8_act as MX
from oracle import nvfp4 as N
from tests.test_oracle_mx_pins import e4m3_py, quant_block_py
from tests.test_oracle_pins import (_py_dequant, _py_ffn, _py_matvec, _tiny_custom,
                                    bf16_from_bits, e2m1_from_bits)


def _forced_sets(L_row, k, rng):
    """Two non-exact selections: ranks 2..k+1, and k experts drawn at random
    (ordered by descending logit, as the GPU reports them)."""
    order = sorted(range(len(L_row)), key=lambda e: (-L_row[e], e))
    shifted = order[1:k + 1]
    drawn = sorted(rng.choice(len(L_row), size=k, replace=False).tolist(),
                   key=lambda e: (-L_row[e], e))
    return [shifted, drawn]


def _py_weights(L_row, ids):
    top = max(L_row[e] for e in ids)
    z = [math.exp(L_row[e] - top) for e in ids]
    s = math.fsum(z)
    return [v / s for v in z]


def _py_token(x_row, ws, experts, shared):
    """shared row, then w_j * y_j in the set's order, summed per element."""
    H = len(x_row)
    terms = [[0.0] * H if shared is None else _py_ffn(x_row, *shared)]
    for w, ex in zip(ws, experts):
        terms.append([w * v for v in _py_ffn(x_row, *ex)])
    return np.array([math.fsum(t[h] for t in terms) for h in range(H)])


def _py_mx_expert(bank, e):
    return (_py_dequant(bank["gate_up_codes"][e, 0], bank["gate_up_scales"][e, 0]),
            _py_dequant(bank["gate_up_codes"][e, 1], bank["gate_up_scales"][e, 1]),
            _py_dequant(bank["down_codes"][e], bank["down_scales"][e]))


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(b)


# ---------------------------------------------------------------------------
# default mode
# ---------------------------------------------------------------------------

def test_token_out_with_exact_ids_reproduces_layer_rows():
    w = S.get("tiny")
    d = S.gen_inputs(w, seed=0)
    for shared in (d["shared"], None):
        r = O.layer(d["x"], d["w_router"], None, d["routed"], shared, w.k)
        for t in range(w.T):
            ysh = None if shared is None else r["y_shared"][t]
            got = O.token_out_with(r["x"], r["logits"], t, r["ids"][t], d["routed"], ysh)
            np.testing.assert_allclose(got, r["out"][t], rtol=1e-12, atol=1e-12)


def test_token_out_with_forced_selection_matches_pure_python():
    w = _tiny_custom()
    d = S.gen_inputs(w, seed=0)
    r = O.route(d["x"], d["w_router"], d["bias"], w.k)
    X = [[bf16_from_bits(b) for b in row] for row in d["x"]]
    WR = [[bf16_from_bits(b) for b in row] for row in d["w_router"]]
    experts = [_py_mx_expert(d["routed"], e) for e in range(w.E)]
    shared = _py_mx_expert(d["shared"], 0)
    y_sh = O.shared_out(r["x"], d["shared"])
    rng = np.random.default_rng(11)
    n_forced = 0
    for t in range(w.T):
        L = _py_matvec(WR, X[t])
        for ids in _forced_sets(L, w.k, rng):
            n_forced += sorted(ids) != sorted(r["ids"][t].tolist())
            ref = _py_token(X[t], _py_weights(L, ids), [experts[e] for e in ids], shared)
            got = O.token_out_with(r["x"], r["logits"], t, ids, d["routed"], y_sh[t])
            assert _rel(got, ref) <= 1e-12, (t, ids)
    assert n_forced >= w.T          # the shifted set is never the exact one


def test_token_out_with_weights_are_renormalised_over_the_forced_set():
    # a set the exact routing would never pick: its weights must still sum to 1
    # (the output is linear in them, so doubling every expert's output must
    # double the routed part exactly)
    w = _tiny_custom()
    d = S.gen_inputs(w, seed=0)
    r = O.route(d["x"], d["w_router"], None, w.k)
    worst = np.argsort(r["logits"][0])[:w.k]            # the k lowest logits
    base = O.token_out_with(r["x"], r["logits"], 0, worst, d["routed"], None)
    b2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d["routed"].items()}
    b2["down_scales"] += 1
    dbl = O.token_out_with(r["x"], r["logits"], 0, worst, b2, None)
    np.testing.assert_array_equal(dbl, 2 * base)
    wts = O.topk_weights(r["logits"][:1], np.asarray(worst)[None, :])[0]
    assert abs(wts.sum() - 1) < 1e-15


# ---------------------------------------------------------------------------
# MXFP8-activation mode
# ---------------------------------------------------------------------------

def _py_round_mx(vals):
    """Round a vector in blocks of 32 with the brute-force block quantiser."""
    out = []
    for b0 in range(0, len(vals), 32):
        codes, s = quant_block_py(vals[b0:b0 + 32])
        out.extend(e4m3_py(c) * math.ldexp(1.0, s - 127) for c in codes)
    return out


def _py_ffn_mx(xq, wg, wu, wd):
    g = _py_matvec(wg, xq)
    u = _py_matvec(wu, xq)
    h = _py_round_mx([gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)])
    return _py_matvec(wd, h)


def test_token_out_with_mx_forced_selection_matches_pure_python():
    w = _tiny_custom()
    d = S.gen_inputs(w, seed=0)
    r = MX.layer_mx(d["x"], d["w_router"], None, d["routed"], d["shared"], w.k)
    X = [[bf16_from_bits(b) for b in row] for row in d["x"]]
    WR = [[bf16_from_bits(b) for b in row] for row in d["w_router"]]
    experts = [_py_mx_expert(d["routed"], e) for e in range(w.E)]
    shared = _py_mx_expert(d["shared"], 0)
    rng = np.random.default_rng(12)
    for t in range(w.T):
        xq = _py_round_mx(X[t])
        np.testing.assert_array_equal(r["xq"][t], xq)
        L = _py_matvec(WR, X[t])                       # routing on the exact x
        sets = _forced_sets(L, w.k, rng) + [r["ids"][t].tolist()]
        for ids in sets:
            ws = _py_weights(L, ids)
            H = len(xq)
            terms = [_py_ffn_mx(xq, *shared)]
            for wj, e in zip(ws, ids):
                terms.append([wj * v for v in _py_ffn_mx(xq, *experts[e])])
            ref = np.array([math.fsum(tt[h] for tt in terms) for h in range(H)])
            got = MX.token_out_with_mx(r["xq"], r["logits"], t, ids, d["routed"], r["y_shared"][t])
            assert _rel(got, ref) <= 1e-12, (t, ids)
        # the exact set reproduces the layer's own row
        np.testing.assert_allclose(
            MX.token_out_with_mx(r["xq"], r["logits"], t, r["ids"][t], d["routed"],
                                 r["y_shared"][t]), r["out"][t], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# NVFP4 experts
# ---------------------------------------------------------------------------

def _py_nv_dequant(codes, scales, gscale):
    Nr, half = codes.shape
    out = []
    for n in range(Nr):
        row = []
        for b in range(half):
            byte = int(codes[n, b])
            for c in (byte & 15, byte >> 4):
                k = len(row)
                sc = int(scales[n, k // 16])
                e, m = (sc >> 3) & 15, sc & 7
                mag = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
                row.append(e2m1_from_bits(c) * (-mag if sc & 0x80 else mag) * gscale)
        out.append(row)
    return out


def _py_nv_expert(bank, e):
    g = [float(v) for v in np.asarray(bank["global_scales"], np.float32)[e]]
    return (_py_nv_dequant(bank["gate_up_codes"][e, 0], bank["gate_up_scales"][e, 0], g[0]),
            _py_nv_dequant(bank["gate_up_codes"][e, 1], bank["gate_up_scales"][e, 1], g[1]),
            _py_nv_dequant(bank["down_codes"][e], bank["down_scales"][e], g[2]))


def test_token_out_with_nvfp4_forced_selection_matches_pure_python():
    w = _tiny_custom()
    d = S.gen_inputs(w, seed=0)
    routed = S.gen_nvfp4_bank(w, 0)
    shared = S.gen_nvfp4_bank(w, 0, shared=True)
    r = N.layer_nvfp4(d["x"], d["w_router"], None, routed, shared, w.k)
    X = [[bf16_from_bits(b) for b in row] for row in d["x"]]
    WR = [[bf16_from_bits(b) for b in row] for row in d["w_router"]]
    experts = [_py_nv_expert(routed, e) for e in range(w.E)]
    sh = _py_nv_expert(shared, 0)
    rng = np.random.default_rng(13)
    for t in range(w.T):
        L = _py_matvec(WR, X[t])
        for ids in _forced_sets(L, w.k, rng) + [r["ids"][t].tolist()]:
            ref = _py_token(X[t], _py_weights(L, ids), [experts[e] for e in ids], sh)
            got = N.token_out_with_nvfp4(r["x"], r["logits"], t, ids, routed, r["y_shared"][t])
            assert _rel(got, ref) <= 1e-12, (t, ids)
