"""Pins of the MXFP8-activation oracle (oracle.mxfp8_act) against things other
than itself: the E4M3 bit-field definition, a brute-force nearest-value
search over all 127 non-negative E4M3 magnitudes, exact round trips of
representable blocks, the rounding error bound, power-of-two equivariance,
and a closed-form identity probe of the whole MX layer.

A plausible mistake in the quantiser (scale exponent off by one, wrong
emax, ties away from zero instead of to even, no clamp at 448, lost sign of
a value that rounds to zero, subnormals flushed) fails one of them.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import moe as O
from oracle import mxfp8_act as M


def e4m3_py(b: int) -> float:
    """E4M3 from its fields, written independently: value = m * 2^-9 for
    exponent field 0, (8 + m) * 2^(e - 10) otherwise; S.1111.111 is NaN."""
    e, m = (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
    return -mag if b & 0x80 else mag


MAGS = [(c, e4m3_py(c)) for c in range(0x7F)]  # every non-negative finite code


def quant_block_py(vals):
    """Brute force of one 32-value block: scale from the binade of the
    largest magnitude minus 8, then the nearest E4M3 magnitude by search
    (ties to the even code), clamped to 448, sign kept."""
    amax = max(abs(v) for v in vals)
    if amax == 0:
        se = -127
    else:
        se = max(-127, min(127, (math.frexp(amax)[1] - 1) - 8))
    X = math.ldexp(1.0, se)
    out = []
    for v in vals:
        q = abs(v) / X
        if q >= 448.0:
            c = 0x7E
        else:
            c = min(MAGS, key=lambda cm: (abs(cm[1] - q), cm[0] & 1))[0]
        out.append(c | (0x80 if math.copysign(1.0, v) < 0 else 0))
    return out, se + 127


def test_e4m3_table_matches_bit_fields_and_named_constants():
    b = np.arange(256)
    got = M.e4m3_to_f64(b)
    for c in range(256):
        ref = e4m3_py(c)
        if math.isnan(ref):
            assert math.isnan(got[c]), c
        else:
            assert got[c] == ref and math.copysign(1, got[c]) == math.copysign(1, ref), c
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xC0] == -2.0
    assert math.isnan(got[0x7F]) and math.isnan(got[0xFF])
    assert np.isfinite(np.delete(got, [0x7F, 0xFF])).all()  # no infinities in E4M3


def _bf16_exact(v):
    """Round fp64 to the nearest bf16 value (the activations are bf16)."""
    f = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    f = (f + 0x7FFF + ((f >> 16) & 1)) >> 16 << 16
    return f.astype(np.uint32).view(np.float32).astype(np.float64)


def _edge_blocks(rng):
    blocks = []
    blocks.append(_bf16_exact(rng.standard_normal(32)))
    blocks.append(_bf16_exact(rng.standard_normal(32) * 1e-3))
    z = np.zeros(32)
    z[5] = -0.0
    blocks.append(z)                                   # all zero, one -0
    b = _bf16_exact(rng.standard_normal(32))
    b[3] = 0.0
    b[4] = -1e-30                                      # rounds to -0
    blocks.append(b)
    b = np.full(32, 1.0)
    b[0] = 1.9375                                      # q = 496 > 448: clamp
    b[1] = 1.8125                                      # q = 464: tie area, clamp
    b[2] = -1.78125                                    # q = 456: rounds to 448
    blocks.append(b)
    # exact midpoints between E4M3 neighbours (ties to even) with X = 1
    b = np.zeros(32)
    b[0] = 256.0
    b[1:9] = [1.0625, 1.1875, 1.3125, 2.125, 2.375, 9 * 2.0 ** -10, 15 * 2.0 ** -10, 0.5 * 2.0 ** -9]
    b[9:13] = [-1.0625, -2.375, 288.0 + 8.0, 304.0 + 8.0]
    blocks.append(b)
    blocks.append(_bf16_exact(rng.standard_normal(32) * 2.0 ** 100))   # large scale
    blocks.append(_bf16_exact(rng.standard_normal(32) * 2.0 ** -125))  # scale clamps at byte 0
    t = np.full(32, 2.0 ** -133)                        # bf16 subnormal amax
    blocks.append(t)
    return blocks


def test_quantise_matches_brute_force_search():
    rng = np.random.default_rng(7)
    blocks = _edge_blocks(rng) + [_bf16_exact(rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20))
                                  for _ in range(24)]
    v = np.stack(blocks)
    codes, scales = M.quantise_mxfp8(v)
    for i, blk in enumerate(blocks):
        ref_codes, ref_scale = quant_block_py([float(t) for t in blk])
        assert scales[i, 0] == ref_scale, i
        assert list(codes[i]) == ref_codes, (i, list(codes[i]), ref_codes)


def test_scale_is_binade_of_amax_minus_eight():
    v = np.zeros((3, 32))
    v[0, 0] = 1.0
    v[1, 0] = 447.0
    v[2, 0] = 0.75
    _, s = M.quantise_mxfp8(v)
    assert list(s[:, 0]) == [127 - 8, 127 + 8 - 8, 127 - 1 - 8]


def test_representable_blocks_round_trip_exactly():
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(0x7F)])
    for _ in range(50):
        c = rng.choice(finite, 32)
        c[rng.integers(0, 32)] = rng.integers(0x78, 0x7F)  # amax in [256, 448]: scale 1
        v = M.e4m3_to_f64(c) * np.where(rng.random(32) < 0.5, -1.0, 1.0)
        v = v * 2.0 ** rng.integers(-30, 30)
        assert np.array_equal(M.round_mxfp8(v[None, :])[0], v)


def test_rounding_error_bound():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-10, 10, (64, 1))
    r = M.round_mxfp8(v)
    _, s = M.quantise_mxfp8(v)
    X = np.repeat(O.e8m0_to_f64(s), 32, axis=1)
    q = np.abs(v) / X
    normal = (q >= 2.0 ** -6) & (q <= 448)
    err = np.abs(r - v)
    assert (err[normal] <= 2.0 ** -4 * np.abs(v[normal]) * (1 + 1e-15)).all()
    assert (err[~normal & (q < 1)] <= 2.0 ** -10 * X[~normal & (q < 1)]).all()
    # the rounding is not a no-op: a fraction of a percent to a few percent
    rel = np.linalg.norm(r - v) / np.linalg.norm(v)
    assert 1e-3 < rel < 5e-2


def test_power_of_two_equivariance():
    rng = np.random.default_rng(9)
    v = _bf16_exact(rng.standard_normal((8, 64)))
    c0, s0 = M.quantise_mxfp8(v)
    c1, s1 = M.quantise_mxfp8(v * 2.0 ** 13)
    assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + 13)


def _identity_bank(n):
    codes = np.zeros((n, n // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = 0x2 if i % 2 == 0 else 0x20  # E2M1 code 2 = 1.0
    sc = np.full((n, n // 32), 127, np.uint8)
    return dict(gate_up_codes=np.stack([codes, codes])[None], gate_up_scales=np.stack([sc, sc])[None],
                down_codes=codes[None], down_scales=sc[None])


def test_identity_probe_closed_form():
    """H = I, identity weights, one expert, top-1: g = u = round(x), so
    out = round(silu(round(x)) * round(x)); with x already representable the
    outer rounding is the only one."""
    n, T = 64, 6
    rng = np.random.default_rng(11)
    c = rng.integers(0, 0x7F, (T, n))
    c[:, 0] = 0x7A
    c[:, 32] = 0x79
    x = M.e4m3_to_f64(c) * np.where(rng.random((T, n)) < 0.5, -1.0, 1.0) * 2.0 ** -7
    xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f64(xb), x)
    bank = _identity_bank(n)
    wr = np.zeros((1, n), np.uint16)
    r = M.layer_mx(xb, wr, None, bank, None, k=1)
    h = x * scipy.special.expit(x) * x
    assert np.array_equal(r["xq"], x)
    np.testing.assert_allclose(r["out"], M.round_mxfp8(h), rtol=1e-14, atol=0)
    # and the exact layer differs from it by the h rounding only
    ex = O.layer(xb, wr, None, bank, None, k=1)["out"]
    np.testing.assert_allclose(ex, h, rtol=1e-14, atol=0)
    assert not np.array_equal(ex, r["out"])
