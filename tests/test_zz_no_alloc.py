"""moe_layer_forward_noalloc: the layer on the library's fixed per-GPU
scratch, for callers that cannot allocate. Through the C ABI it must give
the same results as moe_layer_forward with a caller workspace (the same
kernels run; every sum has a fixed order, so the bits agree), call after
call on the one shared array, with a smaller input after a larger one, and
it must reject a call whose workspace would not fit the array.
"""

import types

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
    M.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _both(w, x_bits, wr_bits, rd, sd):
    """(noalloc out, ids, w) and (workspace out, ids, w) for the same call."""
    x, wr = HP.to_dev(x_bits), HP.to_dev(wr_bits)
    T = x_bits.shape[0]
    res = []
    for noalloc in (True, False):
        out = torch.full((T, w.H), 3.0, dtype=torch.float32, device=HP.dev())
        ids = torch.full((T, w.k), -7, dtype=torch.int32, device=HP.dev())
        wt = torch.full((T, w.k), 3.0, dtype=torch.float32, device=HP.dev())
        if noalloc:
            M.moe_layer_forward_noalloc(x, wr, None, rd, sd, w.k, out, ids, wt)
        else:
            ws = M.workspace(T, w.H, w.I, w.E, w.k, HP.dev())
            M.moe_layer_forward(x, wr, None, rd, sd, w.k, out, ids, wt, ws)
        res.append((_np(out), _np(ids), _np(wt)))
    return res


def _same_bits(a, b):
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def _check_oracle(w, x_bits, wr_bits, routed, shared, got, tol):
    out, ids, wt = got
    ref = O.layer(x_bits, wr_bits, None, routed, shared, w.k)
    alt = HP.check_routing(ref, ids, wt, w.k)
    err = HP.rel_l2(out, HP.reference_rows(ref, routed, shared, ref["tokens"], alt))
    assert err < tol, err


def test_noalloc_matches_workspace_call_larger_then_smaller():
    # a 5-token block, then one token (a smaller input on the same array),
    # then the block again
    blk = S.Workload("blk_five_wide", 98, T=5, H=2048, E=128, k=8, I=768, exp_lo=-6, exp_hi=-3)
    d = S.gen_inputs(blk, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])
    one = S.gen_tokens(blk, 0, call=3, T=1)
    for x_bits in (d["x"], one, d["x"]):
        print(f"noalloc: {x_bits.shape[0]} token(s), H={blk.H}", flush=True)
        na, wsr = _both(blk, x_bits, d["w_router"], rd, sd)
        _same_bits(na, wsr)
        _check_oracle(blk, x_bits, d["w_router"], d["routed"], d["shared"], na, HP.FP32_TOL)


def test_noalloc_real_shape_block_then_decode():
    w5 = S.get("spec5")
    w1 = S.get("decode")
    wr = S.gen_router(w5, 0)
    x5 = S.gen_tokens(w5, 0)
    x1 = S.gen_tokens(w1, 0)
    sel = set()
    for x in (x5, x1):
        r = O.route(x, wr, None, w5.k)
        sel |= set(r["ids"].reshape(-1).tolist())
        for t in range(x.shape[0]):
            if r["margin"][t] <= HP.MARGIN:
                for c in O.near_tie_candidates(r["logits"][t], w5.k):
                    sel |= set(c)
    routed = S.gen_bank(w5, 0, experts=sorted(sel))
    shared = S.gen_bank(w5, 0, shared=True)
    rd, sd = HP.bank_to_dev(routed), HP.bank_to_dev(shared)
    for w, x in ((w5, x5), (w1, x1)):
        print(f"noalloc real shape: {x.shape[0]} token(s)", flush=True)
        na, wsr = _both(w, x, wr, rd, sd)
        _same_bits(na, wsr)
        _check_oracle(w, x, wr, routed, shared, na, HP.FP32_TOL)


def test_noalloc_runs_the_many_token_path_where_it_fits():
    # 40 tokens of the small layer need little scratch: the grouped GEMM runs
    w = S.get("tiny")
    d = S.gen_inputs(w, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])
    x = S.gen_tokens(w, 4, T=40)
    na, wsr = _both(w, x, d["w_router"], rd, sd)
    _same_bits(na, wsr)
    _check_oracle(w, x, d["w_router"], d["routed"], d["shared"], na, HP.GEMM_TOL)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 2048 tokens at the real shape need far more than 16 MiB: rejected with
    # MOE_ERR_WORKSPACE before anything is enqueued
    w = S.get("decode")
    T = 2048
    dev = HP.dev()
    x = torch.zeros((T, w.H), dtype=torch.bfloat16, device=dev)
    wr = torch.zeros((w.E, w.H), dtype=torch.bfloat16, device=dev)
    assert M.moe_workspace_bytes(T, w.H, w.I, w.E, w.k) > 16 << 20
    # a bank struct with aligned non-null addresses: validation reads none of
    # them, and the workspace check fails before any launch
    fake = 0x10000
    rd = types.SimpleNamespace(struct=M.Bank(fake, fake, fake, fake, w.E, w.H, w.I))
    out = torch.full((T, w.H), 3.0, dtype=torch.float32, device=dev)
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward_noalloc(x, wr, None, rd, None, w.k, out)
    assert ei.value.status == M.MOE_ERR_WORKSPACE
    assert M.moe_last_call_launches() == 0
    assert torch.all(out == 3.0)
