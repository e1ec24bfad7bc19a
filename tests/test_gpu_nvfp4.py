"""Parity of the NVFP4 expert path (moe_expert_ffn_nvfp4,
moe_layer_forward_nvfp4) with the fp64 oracle, oracle.nvfp4.

Bars: the weights are dequantised exactly on both sides (E2M1 x E4M3 is
exact in bf16 and fp16), the matrix scale costs one fp32 rounding of each
sum. So the GEMVs (fp32 h) differ from the oracle by fp32 summation only
(FP32_TOL), the grouped GEMM carries h in fp16 (GEMM_TOL), and the layer
takes the routing rules and output bar of the default mode.
"""

import numpy as np
import pytest
import scipy.special

import synthetic as S
from oracle import moe as O
from oracle import nvfp4 as N
from tests import _helpers as HP

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("mxfp4_routed_expert_softmax_amd")

MID = S.Workload("nv_mid", 97, T=300, H=512, E=6, k=2, I=256, exp_lo=-6, exp_hi=-3, zipf_s=1.5)


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


def _names():
    return [M.moe_launch_name(i) for i in range(M.moe_last_call_launches())]


def run_ffn(x_bits, bank_np, offsets, row_token, R):
    T, H = x_bits.shape
    bank = M.NvBankTensors.from_numpy(bank_np, HP.dev())
    y = torch.empty((R, H), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(T, H, bank.I, bank.E, max(1, -(-R // T)), HP.dev())
    off = None if offsets is None else HP.to_dev(np.asarray(offsets, np.int32))
    rt = None if row_token is None else HP.to_dev(np.asarray(row_token, np.int32))
    M.moe_expert_ffn_nvfp4(HP.to_dev(x_bits), bank, off, rt, R, y, ws)
    return _np(y), _names()


@pytest.mark.parametrize("w,tol,kernel", [(S.get("tiny"), HP.FP32_TOL, "gateup_gemv_kernel"),
                                          (MID, HP.GEMM_TOL, "gemm_gateup_kernel")],
                         ids=["gemv", "gemm"])
def test_ffn_bucketed_rows(w, tol, kernel):
    x, wr, bias = S.gen_tokens(w, 1), S.gen_router(w, 1), S.gen_zipf_bias(w, 1)
    bank = S.gen_nvfp4_bank(w, 1)
    r = O.route(x, wr, bias, w.k)
    y, names = run_ffn(x, bank, r["offsets"], r["row_token"], w.R)
    ref = N.expert_rows_nvfp4(r["x"], bank, r["offsets"], r["row_token"])
    err = HP.rel_l2(y, ref)
    print(w.name, names, err)
    assert kernel in names
    assert err < tol


def test_ffn_gemm_buckets_around_sixteen_rows():
    # buckets of at most 16 rows take 16-row tiles with three stages (8 K
    # steps of gate/up: four 2-step scale chunks); 17 rows and more take the
    # 64-row tiles
    w = S.Workload("nv_k8", 98, T=200, H=1024, E=6, k=2, I=512, exp_lo=-6, exp_hi=-3)
    counts = np.array([16, 17, 15, 1, 0, 100])  # 149 rows: above the GEMV path
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    rng = np.random.default_rng([w.cfg_id, 12])
    row_token = rng.integers(0, w.T, R).astype(np.int32)
    x = S.gen_tokens(w, 1)
    bank = S.gen_nvfp4_bank(w, 1)
    y, names = run_ffn(x, bank, offsets, row_token, R)
    assert "gemm_gateup_kernel" in names
    ref = N.expert_rows_nvfp4(O.bf16_to_f64(x), bank, offsets, row_token)
    err = HP.rel_l2(y, ref)
    print(counts.tolist(), err)
    assert err < HP.GEMM_TOL


@pytest.mark.parametrize("T", [4, 300])
def test_ffn_identity_probe(T):
    n = 256
    codes = np.zeros((n, n // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = 0x2 if i % 2 == 0 else 0x20
    sc = np.full((n, n // 16), 0x38, np.uint8)
    bank = dict(gate_up_codes=np.stack([codes, codes])[None], gate_up_scales=np.stack([sc, sc])[None],
                down_codes=codes[None], down_scales=sc[None],
                global_scales=np.array([[2.0, 0.5, 0.25]], np.float32))
    x = S.gen_tokens(S.Workload("eye", 98, T=T, H=n, E=1, k=1, I=n, exp_lo=0, exp_hi=0), 0)
    y, names = run_ffn(x, bank, None, None, T)
    xf = O.bf16_to_f64(x)
    ref = 0.25 * (2 * xf) * scipy.special.expit(2 * xf) * (0.5 * xf)
    assert HP.rel_l2(y, ref) < (HP.FP32_TOL if T <= 128 else HP.GEMM_TOL)


def run_layer(x_bits, wr_bits, bias, routed_np, shared_np, k):
    T = x_bits.shape[0]
    rd = M.NvBankTensors.from_numpy(routed_np, HP.dev())
    sd = None if shared_np is None else M.NvBankTensors.from_numpy(shared_np, HP.dev())
    out = torch.empty((T, rd.H), dtype=torch.float32, device=HP.dev())
    ids = torch.empty((T, k), dtype=torch.int32, device=HP.dev())
    wt = torch.empty((T, k), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(T, rd.H, rd.I, rd.E, k, HP.dev())
    b = None if bias is None else HP.to_dev(bias)
    M.moe_layer_forward_nvfp4(HP.to_dev(x_bits), HP.to_dev(wr_bits), b, rd, sd, k, out, ids, wt, ws)
    HP.assert_waits_ok(ws)
    return _np(out), _np(ids), _np(wt), _names()


def _parity(w, x, wr, bias, routed, shared, tokens=None, tol=HP.OUT_TOL):
    ref = N.layer_nvfp4(x, wr, bias, routed, shared, w.k, tokens=tokens)
    out, ids, wt, names = run_layer(x, wr, bias, routed, shared, w.k)
    tok = ref["tokens"]
    alt = HP.check_routing(ref, ids, wt, w.k)
    rows = [N.token_out_with_nvfp4(ref["x"], ref["logits"], t, alt[t], routed,
                                   None if ref["y_shared"] is None else ref["y_shared"][i])
            if t in alt else ref["out"][i] for i, t in enumerate(tok)]
    err = HP.rel_l2(out[tok], np.stack(rows))
    print(f"{w.name}: rel-L2 {err:.3e} over {len(tok)} tokens; {names}")
    assert err <= tol
    return err


def test_layer_tiny_with_and_without_shared():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    routed = S.gen_nvfp4_bank(w, 0)
    assert _parity(w, d["x"], d["w_router"], None, routed, S.gen_nvfp4_bank(w, 0, shared=True)) \
        < HP.FP32_TOL
    _parity(w, d["x"], d["w_router"], np.linspace(-1, 1, w.E).astype(np.float32), routed, None)


def _selected(w, x, wr):
    r = O.route(x, wr, None, w.k)
    sel = set(r["ids"].reshape(-1).tolist())
    for t in range(x.shape[0]):
        if r["margin"][t] <= HP.MARGIN:
            for c in O.near_tie_candidates(r["logits"][t], w.k):
                sel |= set(c)
    return sorted(sel)


FUSED = ["gateup_fused_kernel"]
BLOCK = ["route_block_kernel", "gateup_block_kernel", "down_block_mfma_kernel"]


@pytest.mark.parametrize("name,T", [("decode", 1), ("spec5", 2), ("spec5", 5), ("spec5", 8),
                                    ("spec5", 9)])
def test_layer_real_shape_few_tokens(name, T):
    # one token takes the fused launch with NVFP4 items, a block of 2..8
    # tokens the block launches (down on the matrix cores), more tokens the
    # three-launch chain
    w = S.get(name)
    x = S.gen_tokens(w, 0, T=T) if T != w.T else S.gen_tokens(w, 0)
    wT = S.Workload(w.name, w.cfg_id, T=T, H=w.H, E=w.E, k=w.k, I=w.I, exp_lo=w.exp_lo,
                    exp_hi=w.exp_hi)
    wr = S.gen_router(w, 0)
    routed = S.gen_nvfp4_bank(w, 0, experts=_selected(wT, x, wr))
    assert _parity(wT, x, wr, None, routed, S.gen_nvfp4_bank(w, 0, shared=True)) < 1e-4
    names = _names()
    if T == 1:
        assert names == FUSED
    elif T <= 8:
        assert names == BLOCK
    else:
        assert "gateup_block_kernel" not in names


# blocks of tokens at shapes where the item counts, the tokens per block
# (the 5- and the 8-token builds) and the rows per slot differ from the real
# shape's; I = 384 is not a multiple of 256 and leaves the block launches
BLOCK_NV = [
    S.Workload("blk_mid", 96, T=3, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
    S.Workload("blk_small7", 97, T=7, H=512, E=32, k=2, I=256, exp_lo=-6, exp_hi=-3),
    S.Workload("blk_wide8", 98, T=8, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3),
    S.Workload("blk_i384", 99, T=4, H=512, E=32, k=4, I=384, exp_lo=-6, exp_hi=-3),
]


@pytest.mark.parametrize("w", BLOCK_NV, ids=lambda w: w.name)
@pytest.mark.parametrize("shared", [True, False], ids=["shared", "no_shared"])
def test_layer_block_launches(w, shared):
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    sh = S.gen_nvfp4_bank(w, 0, shared=True) if shared else None
    bias = None if shared else np.linspace(-1, 1, w.E).astype(np.float32)
    assert _parity(w, x, wr, bias, S.gen_nvfp4_bank(w, 0), sh) < 1e-4
    if w.I % 256 == 0:
        assert _names() == BLOCK
    else:
        assert "down_block_mfma_kernel" not in _names()


ONE_TOKEN_NV = [
    S.Workload("one_mid", 91, T=1, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
    S.Workload("one_small", 92, T=1, H=512, E=32, k=2, I=256, exp_lo=-6, exp_hi=-3),
    S.Workload("one_wide_k", 94, T=1, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3),
]


@pytest.mark.parametrize("w", ONE_TOKEN_NV, ids=lambda w: w.name)
@pytest.mark.parametrize("shared", [True, False], ids=["shared", "no_shared"])
def test_layer_one_token_fused(w, shared):
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    sh = S.gen_nvfp4_bank(w, 0, shared=True) if shared else None
    bias = None if shared else np.linspace(-1, 1, w.E).astype(np.float32)
    assert _parity(w, x, wr, bias, S.gen_nvfp4_bank(w, 0), sh) < 1e-4
    assert _names() == FUSED


def test_layer_gemm_ragged_and_prefill_sampled():
    w = MID
    x, wr, bias = S.gen_tokens(w, 3), S.gen_router(w, 3), S.gen_zipf_bias(w, 3)
    _parity(w, x, wr, bias, S.gen_nvfp4_bank(w, 3), S.gen_nvfp4_bank(w, 3, shared=True),
            tol=HP.GEMM_TOL)
    w = S.get("prefill2k_zipf")
    x, wr, bias = S.gen_tokens(w, 0), S.gen_router(w, 0), S.gen_zipf_bias(w, 0)
    _parity(w, x, wr, bias, S.gen_nvfp4_bank(w, 0), S.gen_nvfp4_bank(w, 0, shared=True),
            tokens=[0, 1, 1024, 2047], tol=HP.GEMM_TOL)


def test_layer_is_bitwise_deterministic():
    w = MID
    x, wr = S.gen_tokens(w, 5), S.gen_router(w, 5)
    routed, shared = S.gen_nvfp4_bank(w, 5), S.gen_nvfp4_bank(w, 5, shared=True)
    a = run_layer(x, wr, None, routed, shared, w.k)
    b = run_layer(x, wr, None, routed, shared, w.k)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_one_token_fused_deterministic_and_garbage_workspace():
    # the fused launches hand data between workgroups through tagged words in
    # the workspace: whatever the workspace held before must not matter
    w = ONE_TOKEN_NV[0]
    x, wr = S.gen_tokens(w, 2), S.gen_router(w, 2)
    rd = M.NvBankTensors.from_numpy(S.gen_nvfp4_bank(w, 2), HP.dev())
    sd = M.NvBankTensors.from_numpy(S.gen_nvfp4_bank(w, 2, shared=True), HP.dev())
    outs = []
    for fill in (None, 0xFF, 0x00):
        ws = M.workspace(w.T, w.H, w.I, w.E, w.k, HP.dev())
        if fill is not None:
            ws.fill_(fill)
        out = torch.empty((w.T, w.H), dtype=torch.float32, device=HP.dev())
        M.moe_layer_forward_nvfp4(HP.to_dev(x), HP.to_dev(wr), None, rd, sd, w.k, out, None, None, ws)
        assert _names() == FUSED
        HP.assert_waits_ok(ws)
        outs.append(_np(out))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint8), outs[0].view(np.uint8))
