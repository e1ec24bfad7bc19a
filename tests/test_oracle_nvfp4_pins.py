"""Pins of the NVFP4 oracle (oracle.nvfp4) against things other than itself:
an element-by-element decode written from the E2M1 and E4M3 field
definitions, the 16-element scale geometry and nibble order, the matrix
scale's linearity, an identity probe with a closed form, and the reduction
to the MXFP4 oracle when every E4M3 scale is a power of two shared by each
pair of 16-blocks.
"""

import math

import numpy as np
import scipy.special

import synthetic as S
from oracle import moe as O
from oracle import nvfp4 as N


def e2m1_py(c):
    s = -1.0 if c & 8 else 1.0
    e, m = (c >> 1) & 3, c & 1
    return s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m))


def e4m3_py(b):
    e, m = (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
    return -mag if b & 0x80 else mag


def test_dequant_matches_elementwise_decode():
    rng = np.random.default_rng(3)
    Nr, K = 8, 64
    codes = rng.integers(0, 256, (Nr, K // 2)).astype(np.uint8)
    sc = rng.integers(0, 0x7F, (Nr, K // 16)).astype(np.uint8)
    got = N.dequant_nvfp4(codes, sc, 0.75)
    for n in range(Nr):
        for k in range(K):
            nib = (codes[n, k // 2] >> (4 * (k % 2))) & 15
            ref = e2m1_py(int(nib)) * e4m3_py(int(sc[n, k // 16])) * 0.75
            assert got[n, k] == ref, (n, k)


def test_scale_geometry_is_16_along_k():
    codes = np.full((1, 32), 0x22, np.uint8)        # every element 1.0
    sc = np.array([[0x38, 0x40, 0x48, 0x30]], np.uint8)  # 1, 2, 4, 0.5
    w = N.dequant_nvfp4(codes, sc)[0]
    assert list(w[[0, 15, 16, 31, 32, 47, 48, 63]]) == [1, 1, 2, 2, 4, 4, 0.5, 0.5]


def test_reduces_to_mxfp4_when_scales_are_shared_powers_of_two():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (16, 64)).astype(np.uint8)
    e = rng.integers(-6, 3, (16, 4))
    mx_scales = (127 + e).astype(np.uint8)
    nv_scales = np.repeat((7 + e) << 3, 2, axis=1).astype(np.uint8)   # E4M3 2^e
    assert np.array_equal(N.dequant_nvfp4(codes, nv_scales), O.dequant_mxfp4(codes, mx_scales))


def test_matrix_scale_is_linear_and_identity_probe():
    n = 64
    codes = np.zeros((n, n // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = 0x2 if i % 2 == 0 else 0x20
    sc = np.full((n, n // 16), 0x38, np.uint8)
    bank = dict(gate_up_codes=np.stack([codes, codes])[None], gate_up_scales=np.stack([sc, sc])[None],
                down_codes=codes[None], down_scales=sc[None],
                global_scales=np.array([[1.0, 1.0, 1.0]], np.float32))
    rng = np.random.default_rng(5)
    xb = S.f64_to_bf16_bits(rng.standard_normal((3, n)))
    x = O.bf16_to_f64(xb)
    y = O.expert_ffn(x, *N.expert_weights_nvfp4(bank, 0))
    np.testing.assert_allclose(y, x * scipy.special.expit(x) * x, rtol=1e-14, atol=0)
    bank["global_scales"] = np.array([[1.0, 0.5, 0.25]], np.float32)
    y2 = O.expert_ffn(x, *N.expert_weights_nvfp4(bank, 0))
    np.testing.assert_allclose(y2, y * 0.125, rtol=1e-14, atol=0)


def test_layer_composition_on_tiny():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    routed = S.gen_nvfp4_bank(w, 0)
    shared = S.gen_nvfp4_bank(w, 0, shared=True)
    r = N.layer_nvfp4(d["x"], d["w_router"], None, routed, shared, w.k)
    for t in range(w.T):
        ref = N.token_out_with_nvfp4(r["x"], r["logits"], t, r["ids"][t], routed, r["y_shared"][t])
        np.testing.assert_allclose(r["out"][t], ref, rtol=1e-12, atol=1e-12)
    assert np.isfinite(r["out"]).all()
    assert N.expert_bytes_nvfp4(5120, 2304) == 3 * 5120 * 2304 * 9 // 16 + 12
