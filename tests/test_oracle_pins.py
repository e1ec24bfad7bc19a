"""Pins of the fp64 oracle against things other than itself.

Each test ties an oracle function to a closed form, an invariant, a special
case with a known answer, a library routine, a brute-force evaluation written
independently in pure Python, or a figure printed on the pages. A plausible
mistake in the oracle (wrong nibble order, wrong E2M1 entry, off-by-one scale
exponent, missing renormalisation, transposed weight, dropped shared expert,
wrong combine index) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special

import synthetic as S
from oracle import moe as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Independent decoders written from the format definitions (OCP MX v1.0)
# ---------------------------------------------------------------------------

def e2m1_from_bits(c: int) -> float:
    """E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent
    field 0 is subnormal with value 0.5 * m."""
    sign = -1.0 if (c >> 3) & 1 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return math.copysign(mag, sign)


def e8m0_from_bits(s: int) -> float:
    return float("nan") if s == 255 else math.ldexp(1.0, s - 127)


def bf16_from_bits(b: int) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


# ---------------------------------------------------------------------------
# C1 / C2: formats
# ---------------------------------------------------------------------------

def test_c1_e2m1_table_matches_bit_fields():
    for c in range(16):
        ref = e2m1_from_bits(c)
        got = O.E2M1_TABLE[c]
        assert got == ref and math.copysign(1, got) == math.copysign(1, ref), c
    # the magnitudes named by the format: 0, 0.5, 1, 1.5, 2, 3, 4, 6
    assert sorted(set(abs(e2m1_from_bits(c)) for c in range(16))) == [0, .5, 1, 1.5, 2, 3, 4, 6]


def test_c1_dequant_nibble_order_and_every_code():
    # one row holding all 256 byte values: element 2b = low nibble, 2b+1 = high
    codes = np.arange(256, dtype=np.uint8)[None, :]          # K = 512
    scales = np.full((1, 16), 127, np.uint8)
    w = O.dequant_mxfp4(codes, scales)[0]
    for b in range(256):
        assert w[2 * b] == e2m1_from_bits(b & 15)
        assert w[2 * b + 1] == e2m1_from_bits(b >> 4)


def test_c1_dequant_scale_per_32_along_k():
    codes = np.full((2, 32), 0x22, np.uint8)                  # every element = 1.0
    scales = np.array([[126, 130], [119, 255]], np.uint8)
    w = O.dequant_mxfp4(codes, scales)
    assert np.all(w[0, :32] == 0.5) and np.all(w[0, 32:] == 8.0)
    assert np.all(w[1, :32] == 2.0 ** -8) and np.all(np.isnan(w[1, 32:]))


def test_c2_e8m0_closed_form():
    s = np.arange(256)
    v = O.e8m0_to_f64(s)
    for i in range(255):
        assert v[i] == e8m0_from_bits(i)
    assert np.isnan(v[255])
    assert v[0] == 2.0 ** -127 and v[127] == 1.0 and v[254] == 2.0 ** 127


def test_bf16_decode_matches_struct():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x8000], np.uint16)
    got = O.bf16_to_f64(bits)
    for b, g in zip(bits, got):
        assert g == bf16_from_bits(b)


def test_generator_bf16_rounding_is_rne():
    # the shared input generator rounds like torch's fp32 -> bf16 cast (RNE)
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(5).normal(0, 3, 4096)
    got = S.f64_to_bf16_bits(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# C3: routing weights
# ---------------------------------------------------------------------------

def _logits(T=64, E=48, seed=1, scale=1.5):
    return np.random.default_rng(seed).normal(0, scale, (T, E))


@pytest.mark.parametrize("k", [1, 2, 6, 48])
def test_c3_weights_sum_to_one_and_equal_renormalised_full_softmax(k):
    L = _logits()
    ids, _ = O.select_topk(L, k)
    w = O.topk_weights(L, ids)
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-15 * k)
    p = scipy.special.softmax(L, axis=1)               # library softmax
    sel = np.take_along_axis(p, ids, axis=1)
    ref = sel / sel.sum(1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-13, atol=0)


def test_c3_topk_is_the_k_largest_in_descending_order():
    L = _logits(T=200, E=384, seed=3)
    ids, _ = O.select_topk(L, 6)
    for t in range(L.shape[0]):
        ref = sorted(range(384), key=lambda e: (-L[t, e], e))[:6]
        assert ids[t].tolist() == ref


def test_margin_is_relative_probability_gap():
    L = _logits(T=32, E=20, seed=4)
    k = 3
    ids, m = O.select_topk(L, k)
    p = scipy.special.softmax(L, axis=1)
    ps = -np.sort(-p, axis=1)
    ref = (ps[:, k - 1] - ps[:, k]) / ps[:, k - 1]
    assert np.allclose(m, ref, rtol=1e-10, atol=1e-15)


def test_near_tie_candidates():
    L = np.array([5.0, 1.0, 3.0, 3.0 + 5e-5, 0.0, 2.9])
    cands = O.near_tie_candidates(L, 2)
    assert cands[0] == (0, 3)
    assert set(cands) == {(0, 3), (0, 2)}
    # a clear margin has one candidate
    assert O.near_tie_candidates(np.array([3.0, 2.0, 1.0]), 1) == [(0,)]


# ---------------------------------------------------------------------------
# C4: bucketing
# ---------------------------------------------------------------------------

def _random_ids(T, E, k, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])


@pytest.mark.parametrize("T,E,k", [(1, 384, 6), (5, 384, 6), (37, 16, 2), (300, 64, 8), (0, 8, 2)])
def test_c4_permute_invariants_and_loops(T, E, k):
    ids = _random_ids(T, E, k, T + E) if T else np.zeros((0, k), np.int64)
    off, rt, inv = O.permute(ids, E)
    off2, rt2, inv2 = O.permute_loops(ids, E)
    assert np.array_equal(off, off2) and np.array_equal(rt, rt2) and np.array_equal(inv, inv2)
    assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), np.bincount(ids.reshape(-1), minlength=E))
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            assert rt[r] == t and off[ids[t, j]] <= r < off[ids[t, j] + 1]
    for e in range(E):                      # stable: tokens ascend in a bucket
        assert np.all(np.diff(rt[off[e]:off[e + 1]]) > 0)
    x = np.random.default_rng(0).normal(size=(T, 3))
    rows = x[rt]                            # scatter to rows, gather back
    assert np.array_equal(rows[inv].reshape(T, k, 3), np.repeat(x[:, None], k, 1))


# ---------------------------------------------------------------------------
# C5 / C6: brute-force dense evaluation in pure Python
# ---------------------------------------------------------------------------

def _tiny_custom(seed=0):
    """A smaller-than-tiny layer so pure-Python loops finish quickly."""
    return S.Workload("brute", 90, T=4, H=64, E=6, k=2, I=32, exp_lo=-3, exp_hi=1,
                      router_std=0.2)


def _py_dequant(codes, scales):
    N, half = codes.shape
    out = []
    for n in range(N):
        row = []
        for b in range(half):
            byte = int(codes[n, b])
            for c in (byte & 15, byte >> 4):
                row.append(e2m1_from_bits(c) * e8m0_from_bits(int(scales[n, len(row) // 32])))
        out.append(row)
    return out


def _py_matvec(W, v):
    return [math.fsum(a * b for a, b in zip(row, v)) for row in W]


def _py_ffn(x, wg, wu, wd):
    g = _py_matvec(wg, x)
    u = _py_matvec(wu, x)
    h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    return _py_matvec(wd, h)


def test_c5_dense_all_experts_with_mask_equals_sparse_oracle():
    w = _tiny_custom()
    d = S.gen_inputs(w, seed=0)
    r = O.layer(d["x"], d["w_router"], d["bias"], d["routed"], d["shared"], w.k)

    X = [[bf16_from_bits(b) for b in row] for row in d["x"]]
    WR = [[bf16_from_bits(b) for b in row] for row in d["w_router"]]
    experts = []
    for bank, e in [(d["routed"], e) for e in range(w.E)] + [(d["shared"], 0)]:
        experts.append((_py_dequant(bank["gate_up_codes"][e, 0], bank["gate_up_scales"][e, 0]),
                        _py_dequant(bank["gate_up_codes"][e, 1], bank["gate_up_scales"][e, 1]),
                        _py_dequant(bank["down_codes"][e], bank["down_scales"][e])))
    for t in range(w.T):
        L = _py_matvec(WR, X[t])
        order = sorted(range(w.E), key=lambda e: (-L[e], e))
        chosen = order[:w.k]
        z = [math.exp(L[e] - L[chosen[0]]) for e in chosen]
        gate = [0.0] * w.E                     # dense mask of routing weights
        for e, zi in zip(chosen, z):
            gate[e] = zi / math.fsum(z)
        terms = [[0.0] * w.H for _ in range(w.E + 1)]
        for e in range(w.E):                   # every expert, masked by its weight
            y = _py_ffn(X[t], *experts[e])
            terms[e] = [gate[e] * v for v in y]
        terms[w.E] = _py_ffn(X[t], *experts[w.E])
        ref = [math.fsum(terms[e][h] for e in range(w.E + 1)) for h in range(w.H)]
        got = r["out"][t]
        err = np.linalg.norm(got - np.array(ref)) / np.linalg.norm(ref)
        assert err <= 1e-12, (t, err)
        assert sorted(r["ids"][t].tolist()) == sorted(chosen)


def test_c6_numpy_oracle_matches_loops_on_tiny_config():
    # the tiny workload itself through a per-element fsum evaluation of one token
    w = S.get("tiny")
    d = S.gen_inputs(w, seed=0)
    r = O.layer(d["x"], d["w_router"], d["bias"], d["routed"], d["shared"], w.k)
    t = 3
    X = [bf16_from_bits(b) for b in d["x"][t]]
    ref = _py_ffn(X, *[_py_dequant(d["shared"][a][0, m] if m is not None else d["shared"][a][0],
                                   d["shared"][b][0, m] if m is not None else d["shared"][b][0])
                       for a, b, m in [("gate_up_codes", "gate_up_scales", 0),
                                       ("gate_up_codes", "gate_up_scales", 1),
                                       ("down_codes", "down_scales", None)]])
    for j, e in enumerate(r["ids"][t]):
        bank = d["routed"]
        y = _py_ffn(X, _py_dequant(bank["gate_up_codes"][e, 0], bank["gate_up_scales"][e, 0]),
                    _py_dequant(bank["gate_up_codes"][e, 1], bank["gate_up_scales"][e, 1]),
                    _py_dequant(bank["down_codes"][e], bank["down_scales"][e]))
        ref = [a + r["w"][t, j] * b for a, b in zip(ref, y)]
    err = np.linalg.norm(r["out"][t] - np.array(ref)) / np.linalg.norm(ref)
    assert err <= 1e-12


# ---------------------------------------------------------------------------
# C7 / C9: special cases
# ---------------------------------------------------------------------------

def test_c7_zero_router_picks_lowest_ids_with_equal_weights():
    w = S.get("tiny")
    x = S.gen_tokens(w, 0)
    wr = np.zeros((w.E, w.H), np.uint16)
    r = O.route(x, wr, None, w.k)
    assert np.all(r["ids"] == np.arange(w.k)[None, :])
    assert np.all(r["w"] == 1.0 / w.k)


def test_c7_bias_only_routing_picks_highest_bias():
    w = S.get("tiny")
    x = np.zeros((3, w.H), np.uint16)
    bias = np.random.default_rng(2).normal(size=w.E).astype(np.float32)
    r = O.route(x, S.gen_router(w, 0), bias, w.k)
    ref = np.argsort(-bias.astype(np.float64), kind="stable")[:w.k]
    assert np.all(r["ids"] == ref[None, :])
    b = bias.astype(np.float64)[ref]
    assert np.allclose(r["w"][0], np.exp(b) / np.exp(b).sum(), rtol=1e-14)


def test_c9_top1_weight_is_exactly_one_and_k_equals_e_is_full_softmax():
    L = _logits(T=16, E=12, seed=7)
    ids, _ = O.select_topk(L, 1)
    assert np.all(O.topk_weights(L, ids) == 1.0)
    ids, m = O.select_topk(L, 12)
    w = O.topk_weights(L, ids)
    p = scipy.special.softmax(L, axis=1)
    assert np.allclose(w, np.take_along_axis(p, ids, axis=1), rtol=1e-13)
    assert np.all(np.isinf(m))


def test_silu_against_library_expit():
    z = np.linspace(-60, 60, 2001)
    assert np.allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# C8: identifiable-constant probes
# ---------------------------------------------------------------------------

def _identity_bank(n: int, scale_gate=127, scale_up=127, scale_down=127):
    """One expert whose three matrices are the n x n identity (code 2 = 1.0)."""
    codes = np.zeros((n, n // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = 0x02 if i % 2 == 0 else 0x20
    sc = lambda v: np.full((n, n // 32), v, np.uint8)  # noqa: E731
    return dict(gate_up_codes=np.stack([codes, codes])[None],
                gate_up_scales=np.stack([sc(scale_gate), sc(scale_up)])[None],
                down_codes=codes[None], down_scales=sc(scale_down)[None], E=1, H=n, I=n)


def test_c8_identity_probe_gives_silu_x_times_x():
    n = 64
    x_bits = S.f64_to_bf16_bits(np.random.default_rng(9).normal(0, 2, (5, n)))
    x = O.bf16_to_f64(x_bits)
    wg, wu, wd = O.expert_weights(_identity_bank(n), 0)
    assert np.array_equal(wg, np.eye(n)) and np.array_equal(wd, np.eye(n))
    y = O.expert_ffn(x, wg, wu, wd)
    assert np.allclose(y, x * x * scipy.special.expit(x), rtol=1e-15, atol=0)


def test_c8_scale_probe_doubles_output_exactly():
    w = S.get("tiny")
    d = S.gen_inputs(w, seed=0)
    x = O.bf16_to_f64(d["x"])
    base = O.expert_ffn(x, *O.expert_weights(d["shared"], 0))
    for which in ("up", "down"):
        b = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d["shared"].items()}
        if which == "up":
            b["gate_up_scales"][0, 1] += 1
        else:
            b["down_scales"][0] += 1
        y = O.expert_ffn(x, *O.expert_weights(b, 0))
        assert np.array_equal(y, 2 * base)


def test_shared_expert_enters_with_weight_one():
    w = S.get("tiny")
    d = S.gen_inputs(w, seed=0)
    with_sh = O.layer(d["x"], d["w_router"], None, d["routed"], d["shared"], w.k)
    without = O.layer(d["x"], d["w_router"], None, d["routed"], None, w.k)
    assert np.allclose(with_sh["out"] - without["out"], with_sh["y_shared"], rtol=1e-13, atol=1e-12)


def test_token_subset_matches_full_layer():
    w = S.get("tiny")
    d = S.gen_inputs(w, seed=0)
    full = O.layer(d["x"], d["w_router"], None, d["routed"], d["shared"], w.k)
    part = O.layer(d["x"], d["w_router"], None, d["routed"], d["shared"], w.k, tokens=[6, 1])
    # BLAS blocks differently for 2 rows than for 8, so allow fp64 rounding
    assert np.allclose(part["out"], full["out"][[6, 1]], rtol=1e-13, atol=1e-11)


# ---------------------------------------------------------------------------
# C10: byte accounting printed on the pages
# ---------------------------------------------------------------------------

def test_c10_byte_accounting_matches_printed_figures():
    g = json.load(open(os.path.join(GOLDEN, "byte_accounting.json")))
    H, I = g["expert_shape"]["H"], g["expert_shape"]["I"]
    b = O.expert_bytes(H, I)
    assert b == 18_800_640
    codes = 3 * H * I // 2
    assert round(codes / 2**20, 2) == g["expert_codes_mib"]["value"]
    assert round(b / 1e6, 2) == g["expert_with_scales_mb"]["value"]
    assert round(b / 2**20, 2) == g["expert_with_scales_mib"]["value"]
    tot = g["routed_total_gib"]
    assert round(tot["layers"] * tot["experts"] * b / 2**30) == tot["value"]
    est = g["v41_decode_estimate"]
    per_token = est["active"] * est["layers"] * b
    assert round(est["bandwidth_gb_s"] * 1e9 / per_token) == est["tok_s"]
