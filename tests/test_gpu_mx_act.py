"""Parity of the MXFP8-activation mode (moe_layer_forward_mxfp8_act,
moe_quantize_mxfp8) with its fp64 oracle, oracle.mxfp8_act.

Bars:
  * the rounding of x: codes and scales bit-exact (the decision is taken on
    exact bf16 values on both sides);
  * routing: the rules of the default mode (it is the same router);
  * outputs: relative L2 error <= MX_TOL against the oracle of the mode.
    Derivation: the products are exact on both sides (E4M3 x E2M1 times
    powers of two), so what remains is fp32 summation and h. g and u are
    fp32 sums of thousands of terms (relative error ~1e-6 to 1e-5 where they
    cancel), so h = silu(g) * u carries ~1e-5; the GPU rounds its fp32 h, the
    oracle its fp64 h, and an element within that distance of a rounding
    midpoint (a chance of about 2e-5 / 2^-3.5, ~2e-4) lands on the
    neighbouring E4M3 value, one step (~9 % of the element) away. Over the I
    terms of a down product that is an rms relative error of about
    sqrt(2e-4) * 0.09 ~ 1.3e-3 at most; measured 3e-5 to 6e-4. MX_TOL = 2e-3.
The error of the mode against the exact layer is printed and bounded loosely
(it is the rounding the mode chooses, a few percent).
"""

import numpy as np
import pytest

import synthetic as S
from oracle import moe as O
from oracle import mxfp8_act as MX
from tests import _helpers as HP

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("mxfp4_routed_expert_softmax_amd")

MX_TOL = 2e-3

# hidden 512 / intermediate 256 with a Zipf-skewed router: one bucket spans
# three 128-row blocks (ragged), several K steps in both GEMMs
GEMM_MID = S.Workload("gemm_mid", 90, T=300, H=512, E=6, k=2, I=256, exp_lo=-6, exp_hi=-3,
                      zipf_s=1.5, desc="grouped-GEMM parity shape")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _edge_rows(rng, H):
    """bf16 rows that exercise the rounding's corners (one block each)."""
    rows = []
    def blk(vals):
        v = np.zeros(32, np.float64)
        v[:len(vals)] = vals
        return v
    specials = [
        blk([]),                                              # all zero
        blk([-0.0, 1e-40, -1e-40]),                           # -0 and bf16 subnormals
        blk([1.9375, 1.8125, -1.78125, 1.0]),                 # clamps at 448
        blk([256.0, 1.0625, 1.1875, 2.375, 9 * 2.0 ** -10, 0.5 * 2.0 ** -9, -1.0625]),  # ties
        blk([3.0e38, -1.0, 1e30]),                            # top of the range
        blk([2.0 ** -126, 2.0 ** -130, -2.0 ** -133]),        # scale clamps at byte 0
    ]
    for s in specials:
        r = rng.standard_normal(H)
        r[:32] = s
        rows.append(r)
    return np.stack(rows)


def _to_bf16_bits(v):
    f = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def test_quantize_mxfp8_bit_exact():
    rng = np.random.default_rng(21)
    H = 320                                   # 10 blocks per row
    v = rng.standard_normal((37, H)) * 2.0 ** rng.integers(-12, 12, (37, 1))
    v = np.concatenate([v, _edge_rows(rng, H)])
    xb = _to_bf16_bits(v)
    T = xb.shape[0]
    x = HP.to_dev(xb)
    codes = torch.empty((T, H), dtype=torch.uint8, device=HP.dev())
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=HP.dev())
    M.moe_quantize_mxfp8(x, codes, scales)
    rc, rs = MX.quantise_mxfp8(O.bf16_to_f64(xb))
    gc, gs = _np(codes), _np(scales)
    assert np.array_equal(gs, rs), np.argwhere(gs != rs)[:5]
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, [(tuple(i), gc[tuple(i)], rc[tuple(i)]) for i in bad[:5]]


def run_layer_mx(x_bits, wr_bits, bias, routed_dev, shared_dev, k):
    T = x_bits.shape[0]
    x, wr = HP.to_dev(x_bits), HP.to_dev(wr_bits)
    b = None if bias is None else HP.to_dev(bias)
    out = torch.empty((T, routed_dev.H), dtype=torch.float32, device=HP.dev())
    ids = torch.empty((T, k), dtype=torch.int32, device=HP.dev())
    wt = torch.empty((T, k), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(T, routed_dev.H, routed_dev.I, routed_dev.E, k, HP.dev())
    M.moe_layer_forward_mxfp8_act(x, wr, b, routed_dev, shared_dev, k, out, ids, wt, ws)
    return _np(out), _np(ids), _np(wt)


def _mx_parity(w, x_bits, wr, bias, routed, shared, tokens=None):
    ref = MX.layer_mx(x_bits, wr, bias, routed, shared, w.k, tokens=tokens)
    out, ids, wt = run_layer_mx(x_bits, wr, bias, HP.bank_to_dev(routed),
                                None if shared is None else HP.bank_to_dev(shared), w.k)
    tok = ref["tokens"]
    alt = HP.check_routing(ref, ids, wt, w.k)
    rows = []
    for i, t in enumerate(tok):
        if t in alt:
            ysh = None if ref["y_shared"] is None else ref["y_shared"][i]
            rows.append(MX.token_out_with_mx(ref["xq"], ref["logits"], t, alt[t], routed, ysh))
        else:
            rows.append(ref["out"][i])
    err = HP.rel_l2(out[tok], np.stack(rows))
    exact = O.layer(x_bits, wr, bias, routed, shared, w.k, tokens=tokens)["out"]
    err_exact = HP.rel_l2(out[tok], exact)
    print(f"{w.name}: rel-L2 {err:.3e} vs the MX oracle, {err_exact:.3e} vs the exact layer, "
          f"{len(tok)} tokens, near-tie swaps {len(alt)}")
    assert np.all(np.isfinite(out[tok]))
    assert err <= MX_TOL
    assert 1e-3 < err_exact < 0.1
    return err


def test_layer_mx_tiny():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    _mx_parity(w, d["x"], d["w_router"], None, d["routed"], d["shared"])


def test_layer_mx_ragged_buckets_with_and_without_shared():
    w = GEMM_MID
    x, wr, bias = S.gen_tokens(w, 3), S.gen_router(w, 3), S.gen_zipf_bias(w, 3)
    routed = S.gen_bank(w, 3)
    shared = S.gen_bank(w, 3, shared=True)
    counts = np.diff(O.route(x, wr, bias, w.k)["offsets"])
    assert counts.max() > 256, counts
    _mx_parity(w, x, wr, bias, routed, shared)
    _mx_parity(w, x, wr, None, routed, None)


def test_layer_mx_few_tokens():
    # the mode runs the grouped GEMM at every T: one token, one ragged block
    w = GEMM_MID
    x, wr = S.gen_tokens(w, 4)[:1], S.gen_router(w, 4)
    _mx_parity(w, x, wr, None, S.gen_bank(w, 4), S.gen_bank(w, 4, shared=True))


@pytest.mark.parametrize("name,tokens", [
    ("prefill2k_zipf", [0, 1, 1024, 2047]),
])
def test_layer_mx_prefill_sampled_tokens(name, tokens):
    w = S.get(name)
    x, wr, bias = S.gen_tokens(w, 0), S.gen_router(w, 0), S.gen_zipf_bias(w, 0)
    _mx_parity(w, x, wr, bias, S.gen_bank(w, 0), S.gen_bank(w, 0, shared=True), tokens=tokens)


def test_layer_mx_is_bitwise_deterministic():
    w = GEMM_MID
    x, wr = S.gen_tokens(w, 5), S.gen_router(w, 5)
    rd, sd = HP.bank_to_dev(S.gen_bank(w, 5)), HP.bank_to_dev(S.gen_bank(w, 5, shared=True))
    a = run_layer_mx(x, wr, None, rd, sd, w.k)
    b = run_layer_mx(x, wr, None, rd, sd, w.k)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_layer_mx_rejects_shapes_outside_its_tiling():
    # H = 160 is a valid layer width but not a multiple of the 256-wide tile
    w = S.Workload("narrow", 91, T=4, H=160, E=4, k=2, I=128, exp_lo=-6, exp_hi=-3)
    bank = HP.bank_to_dev(S.gen_bank(w, 0))
    x = HP.to_dev(S.gen_tokens(w, 0))
    wr = HP.to_dev(S.gen_router(w, 0))
    out = torch.empty((w.T, w.H), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(w.T, w.H, w.I, w.E, w.k, HP.dev())
    with pytest.raises(M.MoeError) as e:
        M.moe_layer_forward_mxfp8_act(x, wr, None, bank, None, w.k, out, None, None, ws)
    assert e.value.status == M.MOE_ERR_UNSUPPORTED
