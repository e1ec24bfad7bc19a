"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every test runs the library on cuda:0 and compares with oracle values
computed on the CPU from the same seeded bits. Sub-steps are compared one by
one (logits, ids, weights, bucketing, per-row expert outputs, the combined
output), not just the final tensor.
"""

import numpy as np
import pytest

import synthetic as S
from oracle import moe as O
from tests import _helpers as HP

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("mxfp4_routed_expert_softmax_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.lib()  # fails loudly when the library is not built
    yield
    torch.cuda.synchronize()


def _np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def run_router(w, x_bits, wr_bits, bias, k=None):
    k = w.k if k is None else k
    T = x_bits.shape[0]
    x, wr = HP.to_dev(x_bits), HP.to_dev(wr_bits)
    b = None if bias is None else HP.to_dev(bias)
    ids = torch.empty((T, k), dtype=torch.int32, device=HP.dev())
    wt = torch.empty((T, k), dtype=torch.float32, device=HP.dev())
    lg = torch.empty((T, w.E), dtype=torch.float32, device=HP.dev())
    M.moe_router_topk(x, wr, b, k, ids, wt, lg, None)
    return _np(lg), _np(ids), _np(wt)


@pytest.mark.parametrize("name", ["tiny", "decode", "spec5", "prefill2k_zipf", "prefill16k"])
def test_router_topk_matches_oracle(name):
    w = S.get(name)
    x = S.gen_tokens(w, 0)
    wr = S.gen_router(w, 0)
    bias = S.gen_zipf_bias(w, 0)
    ref = O.route(x, wr, bias, w.k)
    lg, ids, wt = run_router(w, x, wr, bias)
    L = ref["logits"]
    err = np.abs(lg - L).max() / np.abs(L).max()
    assert err < 1e-5, err
    HP.check_routing(ref, ids, wt, w.k)


@pytest.mark.parametrize("T", [3, 300])
def test_router_topk_many_experts(T):
    # E = 1000: 16 logits per lane in the top-k wave (up to 384: 6); T = 3
    # takes the router GEMV, T = 300 the MFMA router
    w = S.Workload("router_e1000", 94, T=T, H=256, E=1000, k=8, I=128, exp_lo=-6, exp_hi=-3)
    x = S.gen_tokens(w, 0)
    wr = S.gen_router(w, 0)
    ref = O.route(x, wr, None, w.k)
    lg, ids, wt = run_router(w, x, wr, None)
    L = ref["logits"]
    assert np.abs(lg - L).max() / np.abs(L).max() < 1e-5
    HP.check_routing(ref, ids, wt, w.k)


def test_router_zero_weights_tie_to_lowest_ids():
    w = S.get("tiny")
    x = S.gen_tokens(w, 0)
    wr = np.zeros((w.E, w.H), np.uint16)
    for k in (1, 2, w.E):
        _, ids, wt = run_router(w, x, wr, None, k)
        assert np.all(ids == np.arange(k)[None, :])
        assert np.allclose(wt, 1.0 / k, rtol=1e-6)


def test_router_bias_only_and_k_equals_e():
    w = S.get("tiny")
    x = np.zeros((3, w.H), np.uint16)
    bias = np.random.default_rng(2).normal(size=w.E).astype(np.float32)
    ref = O.route(x, S.gen_router(w, 0), bias, w.E)
    _, ids, wt = run_router(w, x, S.gen_router(w, 0), bias, w.E)
    assert np.array_equal(ids, ref["ids"])
    assert np.allclose(wt, ref["w"], atol=1e-6)


# ---------------------------------------------------------------------------
# Bucketing
# ---------------------------------------------------------------------------

def run_permute(ids_np, E):
    T, k = ids_np.shape
    ids = HP.to_dev(ids_np.astype(np.int32))
    off = torch.empty(E + 1, dtype=torch.int32, device=HP.dev())
    rt = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=HP.dev())
    inv = torch.empty((T, k), dtype=torch.int32, device=HP.dev())
    ws = M.workspace(T, 32, 32, E, k, HP.dev())
    M.moe_permute(ids, E, off, rt, inv, ws)
    return _np(off), _np(rt)[: T * k], _np(inv)


@pytest.mark.parametrize("T,E,k", [(1, 384, 6), (5, 384, 6), (8, 16, 2), (341, 384, 6),
                                   (342, 384, 6), (2048, 384, 6), (16384, 384, 6),
                                   (1000, 1024, 8), (37, 1, 1)])
def test_permute_bit_exact(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    off, rt, inv = run_permute(ids, E)
    roff, rrt, rinv = O.permute(ids, E)
    assert np.array_equal(off, roff)
    assert np.array_equal(rt, rrt)
    assert np.array_equal(inv, rinv)


def test_permute_skewed_and_invalid_ids():
    rng = np.random.default_rng(11)
    T, E, k = 3000, 384, 6
    ids = np.stack([np.sort(rng.choice(20, size=k, replace=False))[::-1] for _ in range(T)])
    ids[5, 2] = -1
    ids[2999, 0] = E + 3
    off, rt, inv = run_permute(ids, E)
    valid = (ids >= 0) & (ids < E)
    clean = np.where(valid, ids, 0)
    roff, _, _ = O.permute(clean, E)
    assert off[E] == valid.sum()
    assert inv[5, 2] == -1 and inv[2999, 0] == -1
    # the valid pairs are bucketed exactly as the oracle buckets them alone
    for e in range(E):
        toks = rt[off[e]:off[e + 1]]
        ref_t = [t for t in range(T) if e in ids[t]]
        assert toks.tolist() == ref_t
    for t in range(T):
        for j in range(k):
            if valid[t, j]:
                assert rt[inv[t, j]] == t and off[ids[t, j]] <= inv[t, j] < off[ids[t, j] + 1]


# ---------------------------------------------------------------------------
# Expert FFN
# ---------------------------------------------------------------------------

def run_ffn(x_bits, bank_np, offsets, row_token, R):
    x = HP.to_dev(x_bits)
    bank = HP.bank_to_dev(bank_np)
    off = None if offsets is None else HP.to_dev(np.asarray(offsets, np.int32))
    rt = None if row_token is None else HP.to_dev(np.asarray(row_token, np.int32))
    y = torch.full((max(R, 1), bank.H), float("nan"), dtype=torch.float32, device=HP.dev())
    T = x.shape[0]
    ws = M.workspace(T, bank.H, bank.I, bank.E, max(1, -(-R // T)), HP.dev())
    M.moe_expert_ffn_mxfp4(x, bank, off, rt, R, y, ws)
    HP.assert_waits_ok(ws)
    return _np(y)[:R]


def test_ffn_tiny_rows_match_oracle():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    r = O.route(d["x"], d["w_router"], None, w.k)
    y = run_ffn(d["x"], d["routed"], r["offsets"], r["row_token"], w.R)
    ref = O.expert_rows(r["x"], d["routed"], r["offsets"], r["row_token"])
    for row in range(w.R):
        assert HP.rel_l2(y[row], ref[row]) < 1e-5, row
    ysh = run_ffn(d["x"], d["shared"], None, None, w.T)
    assert HP.rel_l2(ysh, O.shared_out(r["x"], d["shared"])) < 1e-5


def _identity_bank(n, up_codes=None, up_scales=None):
    codes = np.zeros((n, n // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = 0x02 if i % 2 == 0 else 0x20
    one = np.full((n, n // 32), 127, np.uint8)
    uc = codes if up_codes is None else up_codes
    us = one if up_scales is None else up_scales
    return dict(gate_up_codes=np.stack([codes, uc])[None].copy(),
                gate_up_scales=np.stack([one, us])[None].copy(),
                down_codes=codes[None].copy(), down_scales=one[None].copy())


def test_ffn_identity_probe_gives_silu_x_times_x():
    n = 64
    x_bits = S.f64_to_bf16_bits(np.random.default_rng(9).normal(0, 2, (6, n)))
    y = run_ffn(x_bits, _identity_bank(n), None, None, 6)
    x = O.bf16_to_f64(x_bits)
    ref = x * x / (1 + np.exp(-x))
    assert np.allclose(y, ref, rtol=2e-6, atol=1e-30)


def test_ffn_decodes_every_code_and_scale_exactly():
    # gate rows are 1.0 at column k0 and x is one-hot at k0, so g = 1 and
    # h[n] = silu(1) * W_up[n][k0]; down is the identity, so y[n] = h[n].
    n = 256
    rng = np.random.default_rng(3)
    for k0 in (0, 1, 77, 255):
        gate = np.zeros((n, n // 2), np.uint8)
        gate[:, k0 // 2] = 0x02 if k0 % 2 == 0 else 0x20
        up = np.zeros((n, n // 2), np.uint8)
        codes = np.arange(n) % 16
        nib = codes if k0 % 2 == 0 else codes << 4
        up[:, k0 // 2] = nib.astype(np.uint8)
        up_sc = np.full((n, n // 32), 127, np.uint8)
        up_sc[:, k0 // 32] = rng.choice([100, 119, 123, 124, 127, 128, 131, 150], size=n)
        bank = _identity_bank(n, up, up_sc)
        bank["gate_up_codes"][0, 0] = gate
        x = np.zeros((1, n), np.uint16)
        x[0, k0] = 0x3F80  # 1.0
        y = run_ffn(x, bank, None, None, 1)[0]
        ref = O.expert_ffn(O.bf16_to_f64(x), *O.expert_weights(bank, 0))[0]
        vals = O.E2M1_TABLE[codes] * np.ldexp(1.0, up_sc[:, k0 // 32].astype(int) - 127)
        assert np.allclose(ref, vals / (1 + np.exp(-1.0)), rtol=1e-15)
        assert np.allclose(y, ref, rtol=1e-6, atol=0), k0
        assert np.array_equal(np.signbit(y), np.signbit(ref))


def test_ffn_nan_scale_propagates():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    sh = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d["shared"].items()}
    sh["down_scales"][0, 5, 1] = 255
    y = run_ffn(d["x"], sh, None, None, w.T)
    assert np.all(np.isnan(y[:, 5])) and np.all(np.isfinite(np.delete(y, 5, axis=1)))


# ---------------------------------------------------------------------------
# Combine
# ---------------------------------------------------------------------------

def test_combine_fixed_order_matches_oracle():
    rng = np.random.default_rng(4)
    T, k, H = 37, 6, 5120
    R = T * k
    y = rng.normal(size=(R, H)).astype(np.float32)
    inv = rng.permutation(R).reshape(T, k).astype(np.int32)
    wts = rng.random((T, k)).astype(np.float32)
    ysh = rng.normal(size=(T, H)).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.float32, device=HP.dev())
    M.moe_combine(HP.to_dev(y), HP.to_dev(inv), HP.to_dev(wts), HP.to_dev(ysh), out)
    ref = O.combine(y.astype(np.float64), inv, wts.astype(np.float64), ysh.astype(np.float64))
    assert HP.rel_l2(_np(out), ref) < 1e-6
    M.moe_combine(HP.to_dev(y), HP.to_dev(inv), HP.to_dev(wts), None, out)
    assert HP.rel_l2(_np(out), O.combine(y.astype(np.float64), inv, wts.astype(np.float64))) < 1e-6


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def run_layer(x_bits, wr_bits, bias, routed_dev, shared_dev, k):
    T = x_bits.shape[0]
    x, wr = HP.to_dev(x_bits), HP.to_dev(wr_bits)
    b = None if bias is None else HP.to_dev(bias)
    out = torch.empty((T, routed_dev.H), dtype=torch.float32, device=HP.dev())
    ids = torch.empty((T, k), dtype=torch.int32, device=HP.dev())
    wt = torch.empty((T, k), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(T, routed_dev.H, routed_dev.I, routed_dev.E, k, HP.dev())
    M.moe_layer_forward(x, wr, b, routed_dev, shared_dev, k, out, ids, wt, ws)
    HP.assert_waits_ok(ws)
    return _np(out), _np(ids), _np(wt)


def _layer_parity(w, x_bits, wr, bias, routed, shared, tokens=None):
    ref = O.layer(x_bits, wr, bias, routed, shared, w.k, tokens=tokens)
    out, ids, wt = run_layer(x_bits, wr, bias, HP.bank_to_dev(routed),
                             None if shared is None else HP.bank_to_dev(shared), w.k)
    tok = ref["tokens"]
    assert np.isfinite(out).all()          # every row, compared or not
    alt = HP.check_routing(ref, ids, wt, w.k)
    ref_out = HP.reference_rows(ref, routed, shared, tok, alt)
    err = HP.rel_l2(out[tok], ref_out)
    print(f"{w.name}: rel-L2 {err:.3e} over {len(tok)} tokens; near-tie swaps {len(alt)}")
    assert err <= HP.OUT_TOL
    return err


def test_layer_tiny():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    err = _layer_parity(w, d["x"], d["w_router"], None, d["routed"], d["shared"])
    assert err < 1e-5          # fp32 accumulation of exact products


def test_layer_tiny_without_shared_and_with_bias():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    bias = np.linspace(-1, 1, w.E).astype(np.float32)
    _layer_parity(w, d["x"], d["w_router"], bias, d["routed"], None)


def _selected_ids(w, x, wr, bias):
    """Experts the oracle selects, plus every near-tie alternative."""
    r = O.route(x, wr, bias, w.k)
    sel = set(r["ids"].reshape(-1).tolist())
    for t in range(x.shape[0]):
        if r["margin"][t] <= HP.MARGIN:
            for c in O.near_tie_candidates(r["logits"][t], w.k):
                sel |= set(c)
    return sorted(sel)


def _selected_bank(w, x, wr, bias):
    """Bank with only the selected experts generated (others stay zero): the
    layer must read nothing else."""
    sel = _selected_ids(w, x, wr, bias)
    return S.gen_bank(w, 0, experts=sel), sel


@pytest.mark.parametrize("name", ["decode", "spec5", "draft128"])
def test_layer_small_batch_real_shape(name):
    w = S.get(name)
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    routed, sel = _selected_bank(w, x, wr, None)
    shared = S.gen_bank(w, 0, shared=True)
    if w.T > 1:
        print(f"{name} union of routed experts: {len(sel)} of {w.T * w.k}")
    _layer_parity(w, x, wr, None, routed, shared)


def test_layer_decode_token_pool_real_shape():
    # several decode tokens of the benchmark's pool, as independent calls
    w = S.get("decode")
    wr = S.gen_router(w, 0)
    xs = [S.gen_tokens(w, 0, call=c) for c in (1, 2, 3)]
    sel = sorted(set().union(*[_selected_ids(w, x, wr, None) for x in xs]))
    routed = S.gen_bank(w, 0, experts=sel)
    shared = S.gen_bank(w, 0, shared=True)
    for x in xs:
        _layer_parity(w, x, wr, None, routed, shared)
        assert _launches() == ONE_TOKEN_PATH


# One token in one launch, at shapes where the worker count, the shared
# gate/up items per worker (0 to 3), the routed gate/up items per streaming
# workgroup (2, or 3 once 896 workgroups of two no longer cover them, as at
# k = 8 with I = 2304) and the byte-balanced split of the routed rows all
# differ from the real shape's.
ONE_TOKEN = [
    S.Workload("one_mid", 91, T=1, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
    S.Workload("one_small", 92, T=1, H=512, E=32, k=2, I=256, exp_lo=-6, exp_hi=-3),
    S.Workload("one_narrow", 93, T=1, H=256, E=16, k=2, I=256, exp_lo=-6, exp_hi=-3),
    S.Workload("one_wide_k", 94, T=1, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3),
    S.Workload("one_three_items", 104, T=1, H=1024, E=32, k=8, I=2304, exp_lo=-6, exp_hi=-3),
]


def _launches():
    return [M.moe_launch_name(i) for i in range(M.moe_last_call_launches())]


# kernels of the one-token path
ONE_TOKEN_PATH = ["gateup_fused_kernel"]


@pytest.mark.parametrize("variant", ["shared", "no_shared_with_bias"])
@pytest.mark.parametrize("w", ONE_TOKEN, ids=lambda w: w.name)
def test_layer_one_token_path(w, variant):
    d = S.gen_inputs(w, 0)
    bias, shared = None, d["shared"]
    if variant == "no_shared_with_bias":
        bias, shared = np.linspace(-0.5, 0.5, w.E).astype(np.float32), None
    err = _layer_parity(w, d["x"], d["w_router"], bias, d["routed"], shared)
    assert _launches() == ONE_TOKEN_PATH
    assert err < HP.FP32_TOL


# Blocks of 2..5 tokens (verification blocks): router + routing, then the
# streaming gate/up and down launches over the union of the block's experts,
# at shapes where slots hold 1..T tokens, the shared expert's items and the
# per-workgroup item ranges differ from the real shape's.
BLOCKS = [
    S.Workload("blk_small", 95, T=2, H=512, E=32, k=2, I=256, exp_lo=-6, exp_hi=-3),
    S.Workload("blk_mid", 96, T=3, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
    S.Workload("blk_narrow", 97, T=4, H=256, E=16, k=2, I=256, exp_lo=-6, exp_hi=-3),
    S.Workload("blk_five_wide", 98, T=5, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3),
    S.Workload("blk_eight_wide", 101, T=8, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3),
]

# kernels of the block path (2..8 tokens)
def block_path(T):
    return ["route_block_kernel", "gateup_block_kernel", "down_block_mfma_kernel"]


@pytest.mark.parametrize("variant", ["shared", "no_shared_with_bias"])
@pytest.mark.parametrize("w", BLOCKS, ids=lambda w: w.name)
def test_layer_block_path(w, variant):
    d = S.gen_inputs(w, 0)
    bias, shared = None, d["shared"]
    if variant == "no_shared_with_bias":
        bias, shared = np.linspace(-0.5, 0.5, w.E).astype(np.float32), None
    err = _layer_parity(w, d["x"], d["w_router"], bias, d["routed"], shared)
    assert _launches() == block_path(w.T)
    assert err < HP.FP32_TOL


def test_layer_block_of_eight_real_shape():
    # the largest block the streaming path takes, at the real layer shape,
    # correlated tokens as in the verification sweep
    base = S.get("spec5")
    w = S.Workload("verify8", base.cfg_id, T=8, H=base.H, E=base.E, k=base.k, I=base.I,
                   exp_lo=base.exp_lo, exp_hi=base.exp_hi, block=8, noise=base.noise)
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    routed, sel = _selected_bank(w, x, wr, None)
    shared = S.gen_bank(w, 0, shared=True)
    print(f"verify8 union of routed experts: {len(sel)} of {w.T * w.k}")
    err = _layer_parity(w, x, wr, None, routed, shared)
    assert _launches() == block_path(w.T)
    assert err < HP.FP32_TOL


def test_layer_block_of_eight_identical_tokens():
    # every token picks the same experts, so every slot holds 8 tokens: the
    # matrix-core down carries h in two bf16 parts there (16 significant
    # bits) and must stay within the fp32 tolerance
    w = S.Workload("blk_same8", 100, T=8, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3,
                   block=8, noise=0.0)
    d = S.gen_inputs(w, 0)
    r = O.route(d["x"], d["w_router"], None, w.k)
    assert len(set(r["ids"].reshape(-1).tolist())) == w.k  # one set of experts for all
    err = _layer_parity(w, d["x"], d["w_router"], None, d["routed"], d["shared"])
    assert _launches() == block_path(w.T)
    print(f"8 tokens on every slot: rel-L2 {err:.2e}")
    assert err < HP.FP32_TOL


def test_layer_block_path_correlated_tokens_share_experts():
    # tokens drawn as one base plus small noise pick mostly the same
    # experts, so slots hold several tokens each
    w = S.Workload("blk_corr", 99, T=5, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3,
                   block=5, noise=0.05)
    d = S.gen_inputs(w, 0)
    r = O.route(d["x"], d["w_router"], None, w.k)
    union = set(r["ids"].reshape(-1).tolist())
    assert len(union) < w.T * w.k  # experts are shared between tokens
    err = _layer_parity(w, d["x"], d["w_router"], None, d["routed"], d["shared"])
    assert _launches() == block_path(w.T)
    assert err < HP.FP32_TOL


def test_layer_one_token_shapes_share_a_garbage_workspace():
    # one workspace, filled with random bytes, then used by every one-token
    # shape in turn, twice: tags, counters and tables left at other offsets
    # by the previous shape must not matter
    big = ONE_TOKEN[-1]
    ws = M.workspace(1, big.H, big.I, big.E, big.k, HP.dev())
    g = torch.Generator(device=HP.dev()).manual_seed(2)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=HP.dev(), generator=g))
    data = {w.name: S.gen_inputs(w, 0) for w in ONE_TOKEN}
    dev = {w.name: (HP.bank_to_dev(data[w.name]["routed"]), HP.bank_to_dev(data[w.name]["shared"]))
           for w in ONE_TOKEN}
    for _ in range(2):
        for w in ONE_TOKEN:
            d = data[w.name]
            rd, sd = dev[w.name]
            out = torch.empty((1, w.H), dtype=torch.float32, device=HP.dev())
            ids = torch.empty((1, w.k), dtype=torch.int32, device=HP.dev())
            wt = torch.empty((1, w.k), dtype=torch.float32, device=HP.dev())
            M.moe_layer_forward(HP.to_dev(d["x"]), HP.to_dev(d["w_router"]), None, rd, sd, w.k,
                                out, ids, wt, ws)
            assert _launches() == ONE_TOKEN_PATH
            HP.assert_waits_ok(ws)
            ref = O.layer(d["x"], d["w_router"], None, d["routed"], d["shared"], w.k)
            alt = HP.check_routing(ref, _np(ids), _np(wt), w.k)
            err = HP.rel_l2(_np(out), HP.reference_rows(ref, d["routed"], d["shared"],
                                                          ref["tokens"], alt))
            assert err < HP.FP32_TOL, (w.name, err)


def test_layer_one_token_is_bitwise_deterministic():
    w = ONE_TOKEN[0]
    d = S.gen_inputs(w, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])
    a = run_layer(d["x"], d["w_router"], None, rd, sd, w.k)
    b = run_layer(d["x"], d["w_router"], None, rd, sd, w.k)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_layer_is_bitwise_deterministic():
    w = S.get("spec5")
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    routed, _ = _selected_bank(w, x, wr, None)
    rd, sd = HP.bank_to_dev(routed), HP.bank_to_dev(S.gen_bank(w, 0, shared=True))
    a = run_layer(x, wr, None, rd, sd, w.k)
    b = run_layer(x, wr, None, rd, sd, w.k)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("name,tokens", [
    ("prefill2k_zipf", [0, 1, 2, 511, 1024, 1500, 2046, 2047]),
    ("prefill16k", [0, 1, 4097, 8191, 12000, 16383]),
])
def test_layer_prefill_sampled_tokens(name, tokens):
    w = S.get(name)
    x, wr, bias = S.gen_tokens(w, 0), S.gen_router(w, 0), S.gen_zipf_bias(w, 0)
    routed = S.gen_bank(w, 0)
    shared = S.gen_bank(w, 0, shared=True)
    _layer_parity(w, x, wr, bias, routed, shared, tokens=tokens)


# ---------------------------------------------------------------------------
# ABI behaviour on the device
# ---------------------------------------------------------------------------

def test_abi_zero_tokens_is_a_noop_and_small_workspace_is_rejected():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])
    x = HP.to_dev(d["x"])
    wr = HP.to_dev(d["w_router"])
    out = torch.full((w.T, w.H), 3.0, dtype=torch.float32, device=HP.dev())
    ws = M.workspace(w.T, w.H, w.I, w.E, w.k, HP.dev())
    M.moe_layer_forward(x[:0], wr, None, rd, sd, w.k, out[:0], ws=ws)
    assert torch.all(out == 3.0)
    small = ws[:512]
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(x, wr, None, rd, sd, w.k, out, ws=small)
    assert ei.value.status == M.MOE_ERR_WORKSPACE
    assert torch.all(out == 3.0)


# ---------------------------------------------------------------------------
# The persistent few-token kernel: token counts, reused and garbage workspace
# ---------------------------------------------------------------------------

def test_layer_token_counts_share_one_workspace():
    # T from 1 to past the few-token limit, all through one workspace whose
    # flags and tables are left over from the previous (differently shaped) call
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])
    wr = HP.to_dev(d["w_router"])
    ws = M.workspace(64, w.H, w.I, w.E, w.k, HP.dev())
    for T in (1, 2, 3, 5, 6, 7, 8, 15, 16, 17, 40, 3):
        x_bits = S.gen_tokens(w, 5, call=T, T=T)
        out = torch.empty((T, w.H), dtype=torch.float32, device=HP.dev())
        ids = torch.empty((T, w.k), dtype=torch.int32, device=HP.dev())
        wt = torch.empty((T, w.k), dtype=torch.float32, device=HP.dev())
        M.moe_layer_forward(HP.to_dev(x_bits), wr, None, rd, sd, w.k, out, ids, wt, ws)
        HP.assert_waits_ok(ws)
        ref = O.layer(x_bits, d["w_router"], None, d["routed"], d["shared"], w.k)
        alt = HP.check_routing(ref, _np(ids), _np(wt), w.k)
        err = HP.rel_l2(_np(out), HP.reference_rows(ref, d["routed"], d["shared"],
                                                      ref["tokens"], alt))
        # above 16 tokens the layer runs the MFMA grouped GEMM (fp16 h)
        assert err < (HP.FP32_TOL if T <= 16 else HP.GEMM_TOL), (T, err)


@pytest.mark.parametrize("T", [1, 5, 8])
def test_layer_back_to_back_calls_with_new_tokens_share_a_workspace(T):
    # the few-token paths hand values between workgroups as words tagged with
    # the call: a second call on the same workspace, with other tokens, must
    # not take the first call's words (its results would then be the first
    # call's, or a mix)
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])
    wr = HP.to_dev(d["w_router"])
    ws = M.workspace(T, w.H, w.I, w.E, w.k, HP.dev())
    for call in (1, 2, 3):
        x_bits = S.gen_tokens(w, 11, call=call, T=T)
        out = torch.empty((T, w.H), dtype=torch.float32, device=HP.dev())
        ids = torch.empty((T, w.k), dtype=torch.int32, device=HP.dev())
        wt = torch.empty((T, w.k), dtype=torch.float32, device=HP.dev())
        M.moe_layer_forward(HP.to_dev(x_bits), wr, None, rd, sd, w.k, out, ids, wt, ws)
        HP.assert_waits_ok(ws)
        ref = O.layer(x_bits, d["w_router"], None, d["routed"], d["shared"], w.k)
        alt = HP.check_routing(ref, _np(ids), _np(wt), w.k)
        err = HP.rel_l2(_np(out), HP.reference_rows(ref, d["routed"], d["shared"],
                                                      ref["tokens"], alt))
        assert err < HP.FP32_TOL, (T, call, err)


def test_layer_with_garbage_workspace():
    w = S.get("spec5")
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    routed, _ = _selected_bank(w, x, wr, None)
    shared = S.gen_bank(w, 0, shared=True)
    rd, sd = HP.bank_to_dev(routed), HP.bank_to_dev(shared)
    ws = M.workspace(w.T, w.H, w.I, w.E, w.k, HP.dev())
    g = torch.Generator(device=HP.dev()).manual_seed(1)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=HP.dev(), generator=g))
    out = torch.empty((w.T, w.H), dtype=torch.float32, device=HP.dev())
    M.moe_layer_forward(HP.to_dev(x), HP.to_dev(wr), None, rd, sd, w.k, out, ws=ws)
    HP.assert_waits_ok(ws)
    ref = O.layer(x, wr, None, routed, shared, w.k)
    assert HP.rel_l2(_np(out), ref["out"]) < 1e-5


@pytest.mark.parametrize("T,k", [(64, 2), (100, 3)])
def test_ffn_rows_above_the_few_row_path(T, k):
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    x = S.gen_tokens(w, 7, T=T)
    r = O.route(x, d["w_router"], None, k)
    y = run_ffn(x, d["routed"], r["offsets"], r["row_token"], T * k)
    ref = O.expert_rows(r["x"], d["routed"], r["offsets"], r["row_token"])
    assert HP.rel_l2(y, ref) < HP.GEMM_TOL


# ---------------------------------------------------------------------------
# The many-row MFMA grouped GEMM: several row blocks per bucket, ragged
# tails, empty buckets, the shared bucket, every output column
# ---------------------------------------------------------------------------

# hidden 512 / intermediate 256: 2 column tiles of gate/up, 2 of down, 4 K
# steps of gate/up and 2 of down; a Zipf popularity offset on 6 experts makes
# the most popular bucket hold ~300 rows (three 128-row blocks, ragged)
GEMM_MID = S.Workload("gemm_mid", 90, T=300, H=512, E=6, k=2, I=256, exp_lo=-6, exp_hi=-3,
                      zipf_s=1.5, desc="grouped-GEMM parity shape")


def _row_errors(y, ref):
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return num / den


def test_gemm_ffn_routed_buckets_ragged():
    w = GEMM_MID
    x, wr, bias = S.gen_tokens(w, 0), S.gen_router(w, 0), S.gen_zipf_bias(w, 0)
    bank = S.gen_bank(w, 0)
    r = O.route(x, wr, bias, w.k)
    counts = np.diff(r["offsets"])
    assert counts.max() > 256, counts  # three row blocks in one bucket
    y = run_ffn(x, bank, r["offsets"], r["row_token"], w.R)
    ref = O.expert_rows(r["x"], bank, r["offsets"], r["row_token"])
    assert np.all(np.isfinite(y))
    err = _row_errors(y, ref)
    print(f"bucket sizes {counts.tolist()}; max row rel-L2 {err.max():.3e}")
    assert HP.rel_l2(y, ref) < HP.GEMM_TOL
    assert err.max() < 4 * HP.GEMM_TOL


def test_gemm_ffn_hand_made_buckets():
    # bucket sizes around the 128-row block: exactly one block, one block and
    # one row, empty, a single row, two blocks minus one, and a short bucket
    w = GEMM_MID
    counts = np.array([128, 129, 0, 1, 255, 7])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    rng = np.random.default_rng([w.cfg_id, 11])
    row_token = rng.integers(0, w.T, R).astype(np.int32)
    x = S.gen_tokens(w, 1)
    bank = S.gen_bank(w, 1)
    y = run_ffn(x, bank, offsets, row_token, R)
    ref = O.expert_rows(O.bf16_to_f64(x), bank, offsets, row_token)
    assert HP.rel_l2(y, ref) < HP.GEMM_TOL
    assert _row_errors(y, ref).max() < 4 * HP.GEMM_TOL


# hidden 1024 / intermediate 512: 8 K steps of gate/up (two 4-step scale
# chunks), 4 of down
GEMM_K8 = S.Workload("gemm_k8", 91, T=200, H=1024, E=6, k=2, I=512, exp_lo=-6, exp_hi=-3,
                     desc="grouped-GEMM parity shape, 8 K steps")
# hidden 768: 24-byte gate/up scale rows, not a multiple of 16 bytes, so
# gate/up loads its scales per step
GEMM_K6 = S.Workload("gemm_k6", 92, T=200, H=768, E=6, k=2, I=256, exp_lo=-6, exp_hi=-3,
                     desc="grouped-GEMM parity shape, per-step scale loads")
# intermediate 768: down's 24-byte scale rows, 6 K steps
GEMM_I768 = S.Workload("gemm_i768", 93, T=200, H=512, E=6, k=2, I=768, exp_lo=-6, exp_hi=-3,
                       desc="grouped-GEMM parity shape, 6 down K steps")


@pytest.mark.parametrize("w", [GEMM_K8, GEMM_K6, GEMM_I768],
                         ids=["chunked_scales", "per_step_scales", "down_k768"])
def test_gemm_ffn_buckets_around_sixteen_rows(w):
    # buckets of at most 16 rows take 16-row tiles with three stages; 17 rows
    # and more take the 64-row tiles
    counts = np.array([16, 17, 15, 1, 0, 100])  # 149 rows: above the GEMV path
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    rng = np.random.default_rng([w.cfg_id, 12])
    row_token = rng.integers(0, w.T, R).astype(np.int32)
    x = S.gen_tokens(w, 1)
    bank = S.gen_bank(w, 1)
    y = run_ffn(x, bank, offsets, row_token, R)
    assert "gemm_gateup_kernel" in [M.moe_launch_name(i) for i in range(M.moe_last_call_launches())]
    ref = O.expert_rows(O.bf16_to_f64(x), bank, offsets, row_token)
    err = _row_errors(y, ref)
    print(f"buckets {counts.tolist()}: max row rel-L2 {err.max():.3e}")
    assert HP.rel_l2(y, ref) < HP.GEMM_TOL
    assert err.max() < 4 * HP.GEMM_TOL


def test_gemm_ffn_single_expert_identity_rows():
    # the shared-expert form: one-expert bank, no offsets, row r = token r
    w = GEMM_MID
    x = S.gen_tokens(w, 2)
    bank = S.gen_bank(w, 2, shared=True)
    y = run_ffn(x, bank, None, None, w.T)
    ref = O.shared_out(O.bf16_to_f64(x), bank)
    assert HP.rel_l2(y, ref) < HP.GEMM_TOL


def test_gemm_layer_all_tokens():
    w = GEMM_MID
    x, wr, bias = S.gen_tokens(w, 3), S.gen_router(w, 3), S.gen_zipf_bias(w, 3)
    routed = S.gen_bank(w, 3)
    shared = S.gen_bank(w, 3, shared=True)
    err = _layer_parity(w, x, wr, bias, routed, shared)
    assert err < HP.GEMM_TOL
    err = _layer_parity(w, x, wr, None, routed, None)
    assert err < HP.GEMM_TOL



def test_gemm_h_beyond_fp16_range_gives_non_finite_rows_not_wrong_ones():
    # The grouped GEMM carries h = silu(g) * u in fp16. A token scaled up by
    # 2^8 drives |h| past the fp16 maximum: its rows must come out non-finite
    # (never finite and wrong), while a token scaled by 2^3 (|h| still in
    # range) and every other row stay within the GEMM tolerance.
    w = GEMM_MID
    x = S.gen_tokens(w, 4).copy()
    big, mid = 17, 42
    xf = O.bf16_to_f64(x)
    xf[big] *= 2.0 ** 8
    xf[mid] *= 2.0 ** 3
    x = S.f64_to_bf16_bits(xf)              # exact: powers of two
    bank = S.gen_bank(w, 4)
    r = O.route(x, S.gen_router(w, 4), S.gen_zipf_bias(w, 4), w.k)
    off, rt = r["offsets"], r["row_token"]
    y = run_ffn(x, bank, off, rt, w.R)
    ref = O.expert_rows(r["x"], bank, off, rt)
    hmax = np.zeros(w.R)
    for e in range(w.E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size:
            wg, wu, _ = O.expert_weights(bank, e)
            X = r["x"][rt[rows]]
            hmax[rows] = np.abs(O.silu(X @ wg.T) * (X @ wu.T)).max(axis=1)
    over = hmax >= 65520.0                  # rounds to inf in fp16
    assert over[rt == big].all() and not over[rt != big].any(), hmax[rt == big]
    assert hmax[rt == mid].max() > 1000.0   # large, but inside the range
    assert not np.isfinite(y[over]).any()
    ok = ~over
    assert np.isfinite(y[ok]).all()
    assert HP.rel_l2(y[ok], ref[ok]) < HP.GEMM_TOL
    assert _row_errors(y[ok], ref[ok]).max() < 4 * HP.GEMM_TOL


# ---------------------------------------------------------------------------
# Fallback kernels for shapes the tiled kernels do not take
# ---------------------------------------------------------------------------

def test_router_unstaged_mfma_kernel_for_hidden_not_multiple_of_64():
    # T > 16 takes the MFMA router; with H % 64 != 0 its unstaged form
    w = S.Workload("rt_h96", 106, T=40, H=96, E=48, k=4, I=64, exp_lo=-6, exp_hi=-3,
                   router_std=0.2)
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    ref = O.route(x, wr, None, w.k)
    lg, ids, wt = run_router(w, x, wr, None)
    assert _launches()[0] == "router_mfma_kernel"
    assert np.abs(lg - ref["logits"]).max() / np.abs(ref["logits"]).max() < 1e-5
    HP.check_routing(ref, ids, wt, w.k)


def test_router_staged_mfma_kernel_is_named_apart():
    w = S.get("prefill2k_zipf")
    x, wr = S.gen_tokens(w, 0)[:64], S.gen_router(w, 0)
    ref = O.route(x, wr, None, w.k)
    lg, ids, wt = run_router(w, x, wr, None)
    assert _launches()[0] == "router_mfma_lds_kernel"
    HP.check_routing(ref, ids, wt, w.k)


def test_layer_gemv_fallback_for_shapes_the_gemm_does_not_tile():
    # 40 tokens with H % 256 != 0 and I % 128 != 0: the bucketed GEMVs (fp32 h)
    # and the unstaged router
    w = S.Workload("gemv_fb", 107, T=40, H=288, E=8, k=4, I=160, exp_lo=-6, exp_hi=-3)
    d = S.gen_inputs(w, 0)
    err = _layer_parity(w, d["x"], d["w_router"], None, d["routed"], d["shared"])
    names = _launches()
    assert "gateup_gemv_kernel" in names and "down_gemv_kernel" in names, names
    assert "router_mfma_kernel" in names, names
    assert err < HP.FP32_TOL


def test_layer_one_token_chain_for_hidden_not_multiple_of_128():
    # one token with H % 128 != 0: the three-launch chain instead of the fused
    # launches
    w = S.Workload("one_h96", 108, T=1, H=96, E=16, k=2, I=64, exp_lo=-6, exp_hi=-3)
    d = S.gen_inputs(w, 0)
    err = _layer_parity(w, d["x"], d["w_router"], None, d["routed"], d["shared"])
    assert _launches() == ["route_kernel", "gateup_kernel", "down_kernel"]
    assert err < HP.FP32_TOL


def test_ffn_few_rows_real_decode_shape_through_its_table_kernel():
    # moe_expert_ffn_mxfp4 with the six rows of one decode token at the real
    # shape: the few-row path (its slot-table kernel, then gate/up and down)
    w = S.get("decode")
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    r = O.route(x, wr, None, w.k)
    bank = S.gen_bank(w, 0, experts=sorted(set(r["ids"][0].tolist())))
    y = run_ffn(x, bank, r["offsets"], r["row_token"], w.k)
    assert _launches() == ["ffn_table_kernel", "gateup_kernel", "down_kernel"]
    ref = O.expert_rows(r["x"], bank, r["offsets"], r["row_token"])
    assert HP.rel_l2(y, ref) < HP.FP32_TOL
