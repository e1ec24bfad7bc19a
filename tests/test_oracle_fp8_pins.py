"""Pins of the FP8 (32 x 32 block-scaled) expert oracle, oracle.fp8_dense,
against things other than itself: an element-by-element decode written from
the E4M3 and E8M0 field definitions, the block geometry (a scale changes
exactly at multiples of 32 in both dimensions, which the 128 x 128 reading
the pages warn about would not), closed forms of an identity probe and a
scale probe, NaN scales, and the layer's composition.
"""

import math

import numpy as np
import scipy.special

import synthetic as S
from oracle import fp8_dense as F
from oracle import moe as O


def e4m3_py(b: int) -> float:
    e, m = (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
    return -mag if b & 0x80 else mag


def test_dequant_matches_elementwise_field_decode():
    rng = np.random.default_rng(1)
    N, K = 64, 96
    w = rng.integers(0, 256, (N, K)).astype(np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x11
    s = rng.integers(118, 136, (N // 32, K // 32)).astype(np.uint8)
    got = F.dequant_fp8_block32(w, s)
    for n in range(N):
        for k in range(K):
            ref = e4m3_py(int(w[n, k])) * math.ldexp(1.0, int(s[n // 32, k // 32]) - 127)
            assert got[n, k] == ref and math.copysign(1, got[n, k]) == math.copysign(1, ref)


def test_scale_blocks_are_32_by_32():
    N, K = 256, 256
    w = np.full((N, K), 0x38, np.uint8)                       # every element 1.0
    s = (120 + (np.arange(64).reshape(8, 8) % 13)).astype(np.uint8)
    W = F.dequant_fp8_block32(w, s)
    assert np.array_equal(W, np.ldexp(1.0, np.repeat(np.repeat(s.astype(int) - 127, 32, 0), 32, 1)))
    # the value changes at row 32 and at column 32, inside what a 128 x 128
    # block would be
    assert W[31, 0] != W[32, 0] and W[0, 31] != W[0, 32]
    assert W[0, 0] == W[31, 31]


def test_nan_scale_propagates():
    w = np.full((32, 32), 0x38, np.uint8)
    assert np.isnan(F.dequant_fp8_block32(w, np.array([[255]], np.uint8))).all()


def _identity_fp8_bank(n, down_scale=127):
    eye = np.where(np.eye(n, dtype=bool), 0x38, 0).astype(np.uint8)
    sc = np.full((n // 32, n // 32), 127, np.uint8)
    return dict(gate_up_w=np.stack([eye, eye])[None], gate_up_scales=np.stack([sc, sc])[None],
                down_w=eye[None], down_scales=np.full((n // 32, n // 32), down_scale, np.uint8)[None],
                E=1, H=n, I=n)


def test_identity_probe_and_scale_probe():
    n = 64
    rng = np.random.default_rng(2)
    x = S.f64_to_bf16_bits(rng.standard_normal((5, n)))
    xf = O.bf16_to_f64(x)
    y = F.dense_ffn_fp8(xf, _identity_fp8_bank(n))
    np.testing.assert_allclose(y, xf * scipy.special.expit(xf) * xf, rtol=1e-14, atol=0)
    y2 = F.dense_ffn_fp8(xf, _identity_fp8_bank(n, down_scale=128))
    assert np.array_equal(y2, 2 * y)


def test_layer_adds_the_fp8_shared_expert_with_weight_one():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    sh = S.gen_fp8_bank(w, 0)
    r = F.layer_fp8_shared(d["x"], d["w_router"], None, d["routed"], sh, w.k)
    base = O.layer(d["x"], d["w_router"], None, d["routed"], None, w.k)
    np.testing.assert_allclose(r["out"], base["out"] + F.dense_ffn_fp8(base["x"], sh),
                               rtol=1e-12, atol=1e-12)
    # zero routed bank: only the shared expert remains
    zero = {k: (np.zeros_like(v) if isinstance(v, np.ndarray) else v) for k, v in d["routed"].items()}
    eye = _identity_fp8_bank(w.H) if w.H == w.I else None
    if eye is not None:
        r0 = F.layer_fp8_shared(d["x"], d["w_router"], None, zero, eye, w.k)
        np.testing.assert_allclose(r0["out"], r0["x"] * scipy.special.expit(r0["x"]) * r0["x"])


def test_expert_bytes_fp8():
    # one byte per weight and one scale byte per 32 x 32 block
    assert F.expert_bytes_fp8(5120, 2304) == 3 * 5120 * 2304 + 3 * 160 * 72
