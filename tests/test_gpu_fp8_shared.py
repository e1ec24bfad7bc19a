"""Parity of the FP8 expert (E4M3 with 32 x 32 ue8m0 block scales) and of the
layer with an FP8 shared expert (moe_expert_ffn_fp8,
moe_layer_forward_fp8_shared) with the fp64 oracle, oracle.fp8_dense.

Bars: the weights are dequantised exactly on both sides, so the few-token
GEMVs (fp32 h) differ from the oracle by fp32 summation only (FP32_TOL);
the grouped GEMM carries h in fp16 (GEMM_TOL, derived in tests/_helpers.py);
the layer takes the routing rules and the output bar of the default mode.
"""

import numpy as np
import pytest
import scipy.special

import synthetic as S
from oracle import fp8_dense as F
from oracle import moe as O
from tests import _helpers as HP

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("mxfp4_routed_expert_softmax_amd")


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


def _launch_names():
    return [M.moe_launch_name(i) for i in range(M.moe_last_call_launches())]


def run_fp8_ffn(x_bits, bank_np):
    T, H = x_bits.shape
    bank = M.Fp8BankTensors.from_numpy(bank_np, HP.dev())
    y = torch.empty((T, H), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(T, H, bank.I, 1, 1, HP.dev())
    M.moe_expert_ffn_fp8(HP.to_dev(x_bits), bank, y, ws)
    names = _launch_names()
    return _np(y), names


SMALL = S.Workload("fp8_small", 95, T=300, H=512, E=4, k=2, I=256, exp_lo=-6, exp_hi=-3)


def _eye_bank(n):
    eye = np.where(np.eye(n, dtype=bool), 0x38, 0).astype(np.uint8)
    sc = np.full((n // 32, n // 32), 127, np.uint8)
    return dict(gate_up_w=np.stack([eye, eye])[None], gate_up_scales=np.stack([sc, sc])[None],
                down_w=eye[None], down_scales=sc[None], E=1, H=n, I=n)


@pytest.mark.parametrize("T", [1, 16, 40])
def test_fp8_ffn_identity_probe(T):
    n = 256
    x = S.gen_tokens(S.Workload("eye", 96, T=T, H=n, E=1, k=1, I=n, exp_lo=0, exp_hi=0), 0)
    y, names = run_fp8_ffn(x, _eye_bank(n))
    xf = O.bf16_to_f64(x)
    ref = xf * scipy.special.expit(xf) * xf
    tol = HP.FP32_TOL if T <= 16 else HP.GEMM_TOL
    print(T, names, HP.rel_l2(y, ref))
    assert HP.rel_l2(y, ref) < tol
    assert ("gemm_fp8w_gateup_kernel" in names) == (T > 16)


@pytest.mark.parametrize("T", [1, 5, 16])
def test_fp8_ffn_every_code_few_tokens(T):
    # all 254 finite E4M3 bytes, subnormals included, through the GEMVs
    w = S.get("tiny")
    bank = S.gen_fp8_bank(w, 1, all_codes=True)
    x = S.gen_tokens(w, 1, T=T)
    y, _ = run_fp8_ffn(x, bank)
    ref = F.dense_ffn_fp8(O.bf16_to_f64(x), bank)
    assert HP.rel_l2(y, ref) < HP.FP32_TOL


@pytest.mark.parametrize("T", [17, 300])
def test_fp8_ffn_gemm_rows(T):
    w = SMALL
    bank = S.gen_fp8_bank(w, 2)
    x = S.gen_tokens(w, 2, T=T)
    y, names = run_fp8_ffn(x, bank)
    ref = F.dense_ffn_fp8(O.bf16_to_f64(x), bank)
    err = HP.rel_l2(y, ref)
    rows = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    print(T, names, err, rows.max())
    assert "gemm_fp8w_down_kernel" in names
    assert err < HP.GEMM_TOL and rows.max() < 4 * HP.GEMM_TOL


def run_layer_fp8(x_bits, wr_bits, bias, routed_dev, shared_dev, k):
    T = x_bits.shape[0]
    out = torch.empty((T, routed_dev.H), dtype=torch.float32, device=HP.dev())
    ids = torch.empty((T, k), dtype=torch.int32, device=HP.dev())
    wt = torch.empty((T, k), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(T, routed_dev.H, routed_dev.I, routed_dev.E, k, HP.dev())
    b = None if bias is None else HP.to_dev(bias)
    M.moe_layer_forward_fp8_shared(HP.to_dev(x_bits), HP.to_dev(wr_bits), b, routed_dev,
                                   shared_dev, k, out, ids, wt, ws)
    HP.assert_waits_ok(ws)
    names = _launch_names()
    return _np(out), _np(ids), _np(wt), names


def _fp8_layer_parity(w, x, wr, bias, routed, shared8, tokens=None, tol=HP.OUT_TOL):
    ref = F.layer_fp8_shared(x, wr, bias, routed, shared8, w.k, tokens=tokens)
    out, ids, wt, names = run_layer_fp8(x, wr, bias, HP.bank_to_dev(routed),
                                        M.Fp8BankTensors.from_numpy(shared8, HP.dev()), w.k)
    tok = ref["tokens"]
    alt = HP.check_routing(ref, ids, wt, w.k)
    rows = []
    for i, t in enumerate(tok):
        rows.append(O.token_out_with(ref["x"], ref["logits"], t, alt[t], routed, ref["y_shared"][i])
                    if t in alt else ref["out"][i])
    err = HP.rel_l2(out[tok], np.stack(rows))
    print(f"{w.name}: rel-L2 {err:.3e} over {len(tok)} tokens; launches {names}")
    assert err <= tol
    return err, names


def test_layer_fp8_shared_tiny():
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    err, _ = _fp8_layer_parity(w, d["x"], d["w_router"], None, d["routed"], S.gen_fp8_bank(w, 0))
    assert err < HP.FP32_TOL


def _selected_bank(w, x, wr, bias):
    r = O.route(x, wr, bias, w.k)
    sel = set(r["ids"].reshape(-1).tolist())
    for t in range(x.shape[0]):
        if r["margin"][t] <= HP.MARGIN:
            for c in O.near_tie_candidates(r["logits"][t], w.k):
                sel |= set(c)
    return S.gen_bank(w, 0, experts=sorted(sel))


BLOCK_PATH = ["route_block_kernel", "gateup_block_kernel", "down_block_mfma_kernel"]


@pytest.mark.parametrize("name,T,path", [
    ("decode", 1, "gateup_fused_kernel"),
    ("spec5", 2, "gateup_block_kernel"),
    ("spec5", 5, "gateup_block_kernel"),
    ("spec5", 6, "gateup_block_kernel"),
    ("spec5", 8, "gateup_block_kernel"),
    ("spec5", 9, "gateup_kernel"),
])
def test_layer_fp8_shared_real_shape_few_tokens(name, T, path):
    # one token streams the FP8 expert inside the fused launch and a block of
    # 2..8 tokens inside the block launches (gate/up in the route launch,
    # down in the gate/up launch's tail); more tokens run it first, in its
    # own two launches
    w = S.get(name)
    x = S.gen_tokens(w, 0, T=T) if T != w.T else S.gen_tokens(w, 0)
    wr = S.gen_router(w, 0)
    wT = S.Workload(w.name, w.cfg_id, T=T, H=w.H, E=w.E, k=w.k, I=w.I, exp_lo=w.exp_lo,
                    exp_hi=w.exp_hi)
    routed = _selected_bank(wT, x, wr, None)
    err, names = _fp8_layer_parity(wT, x, wr, None, routed, S.gen_fp8_bank(w, 0))
    if T == 1:
        assert names == ["gateup_fused_kernel"]
    elif T <= 8:
        assert names == BLOCK_PATH
    else:
        assert names[:2] == ["fp8_gateup_gemv_kernel", "fp8_down_gemv_kernel"]
    assert path in names
    assert err < 1e-4


# blocks of tokens through the block launches at shapes where the item
# counts, the tokens per block and the routed rows per slot differ from the
# real shape's (block of 3: the 5-token build; 7: the 8-token build; every
# finite E4M3 byte in the last)
BLOCK_FP8 = [
    (S.Workload("blk_mid", 96, T=3, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3), False),
    (S.Workload("blk_small7", 97, T=7, H=512, E=32, k=2, I=256, exp_lo=-6, exp_hi=-3), False),
    (S.Workload("blk_wide4", 98, T=4, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3), True),
]


@pytest.mark.parametrize("w,every", BLOCK_FP8, ids=lambda v: getattr(v, "name", str(v)))
def test_layer_fp8_shared_block_launches(w, every):
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    err, names = _fp8_layer_parity(w, x, wr, None, S.gen_bank(w, 0),
                                   S.gen_fp8_bank(w, 0, all_codes=every))
    assert names == BLOCK_PATH
    assert err < 1e-4


# one token through the fused launches at shapes where the item counts and
# the split of the routed rows differ from the real shape's
ONE_TOKEN_FP8 = [
    S.Workload("one_mid", 91, T=1, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
    S.Workload("one_small", 92, T=1, H=512, E=32, k=2, I=256, exp_lo=-6, exp_hi=-3),
    S.Workload("one_wide_k", 94, T=1, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3),
]


@pytest.mark.parametrize("w", ONE_TOKEN_FP8, ids=lambda w: w.name)
def test_layer_fp8_shared_one_token_fused(w):
    x, wr = S.gen_tokens(w, 0), S.gen_router(w, 0)
    err, names = _fp8_layer_parity(w, x, wr, None, S.gen_bank(w, 0), S.gen_fp8_bank(w, 0))
    assert names == ["gateup_fused_kernel"]
    assert err < 1e-4


def test_layer_fp8_shared_one_token_every_code():
    # all finite E4M3 bytes (subnormals included) through the fused items
    w = ONE_TOKEN_FP8[0]
    x, wr = S.gen_tokens(w, 1), S.gen_router(w, 1)
    err, names = _fp8_layer_parity(w, x, wr, None, S.gen_bank(w, 1),
                                   S.gen_fp8_bank(w, 1, all_codes=True))
    assert names == ["gateup_fused_kernel"]
    assert err < 1e-4


def test_layer_fp8_shared_prefill_sampled_tokens():
    w = S.get("prefill2k_zipf")
    x, wr, bias = S.gen_tokens(w, 0), S.gen_router(w, 0), S.gen_zipf_bias(w, 0)
    err, names = _fp8_layer_parity(w, x, wr, bias, S.gen_bank(w, 0), S.gen_fp8_bank(w, 0),
                                   tokens=[0, 1, 1024, 2047], tol=HP.GEMM_TOL)
    assert "gemm_fp8w_gateup_kernel" in names


def test_layer_fp8_shared_is_bitwise_deterministic():
    w = SMALL
    x, wr = S.gen_tokens(w, 5), S.gen_router(w, 5)
    rd = HP.bank_to_dev(S.gen_bank(w, 5))
    sd = M.Fp8BankTensors.from_numpy(S.gen_fp8_bank(w, 5), HP.dev())
    a = run_layer_fp8(x, wr, None, rd, sd, w.k)
    b = run_layer_fp8(x, wr, None, rd, sd, w.k)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_layer_fp8_shared_one_token_deterministic_and_garbage_workspace():
    w = ONE_TOKEN_FP8[0]
    x, wr = S.gen_tokens(w, 2), S.gen_router(w, 2)
    rd = HP.bank_to_dev(S.gen_bank(w, 2))
    sd = M.Fp8BankTensors.from_numpy(S.gen_fp8_bank(w, 2), HP.dev())
    outs = []
    for fill in (None, 0xFF, 0x00):
        ws = M.workspace(w.T, w.H, w.I, w.E, w.k, HP.dev())
        if fill is not None:
            ws.fill_(fill)
        out = torch.empty((w.T, w.H), dtype=torch.float32, device=HP.dev())
        M.moe_layer_forward_fp8_shared(HP.to_dev(x), HP.to_dev(wr), None, rd, sd, w.k, out, None,
                                       None, ws)
        assert _launch_names() == ["gateup_fused_kernel"]
        HP.assert_waits_ok(ws)
        outs.append(_np(out))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint8), outs[0].view(np.uint8))
