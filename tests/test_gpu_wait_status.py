"""A bounded in-kernel wait that gives up must show in the call's results.

The few-token paths hand data between workgroups of one launch and wait for
it with a bounded number of polls. A correct run never exhausts them; if one
did, the call would go on with clamped indices, so the failure must be
visible: the call's last launch writes NaN to every output element, -1 to
the ids and NaN to the weights, and moe_workspace_status reports
MOE_ERR_TIMEOUT. The condition is forced from the host through the test
hook moe_set_wait_test: the routing's first wait then expects a tag that no
word carries and gives up after a few polls, while every other wait and
kernel runs as usual, so every launch still ends normally. A normal call on
the same workspace afterwards must be correct again and report MOE_OK.
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
    M.lib()
    yield
    M.moe_set_wait_test(False)
    torch.cuda.synchronize()


def _names():
    return [M.moe_launch_name(i) for i in range(M.moe_last_call_launches())]


# one workload per few-token path: one token (fused launches), a
# verification block, and the three-launch chain (9 tokens)
PATHS = [
    ("one_token", S.Workload("one_mid", 91, T=1, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
     ["gateup_fused_kernel"]),
    ("block", S.Workload("blk_mid", 96, T=3, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
     ["route_block_kernel", "gateup_block_kernel", "down_block_mfma_kernel"]),
    ("chain", S.Workload("chain9", 105, T=9, H=1024, E=64, k=4, I=512, exp_lo=-6, exp_hi=-3),
     ["route_kernel", "gateup_kernel", "down_kernel"]),
]


def _call(fn, w, d, rd, sd, ws):
    out = torch.full((w.T, w.H), 7.0, dtype=torch.float32, device=HP.dev())
    ids = torch.full((w.T, w.k), 5, dtype=torch.int32, device=HP.dev())
    wt = torch.full((w.T, w.k), 0.5, dtype=torch.float32, device=HP.dev())
    fn(HP.to_dev(d["x"]), HP.to_dev(d["w_router"]), None, rd, sd, w.k, out, ids, wt, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), wt.cpu().numpy()


def _forced_then_normal(fn, w, d, rd, sd, path, ref_fn):
    """ref_fn() -> (oracle layer dict, rows(alt) giving the oracle rows for
    the GPU's selection on near-tie tokens)."""
    ws = M.workspace(w.T, w.H, w.I, w.E, w.k, HP.dev())
    print(f"forced timeout: {w.name} {fn.__name__}", flush=True)
    M.moe_set_wait_test(True)
    try:
        out, ids, wt = _call(fn, w, d, rd, sd, ws)
    finally:
        M.moe_set_wait_test(False)
    assert _names() == path
    assert M.moe_workspace_status(ws) == M.MOE_ERR_TIMEOUT
    assert np.isnan(out).all()
    assert (ids == -1).all()
    assert np.isnan(wt).all()
    # the same workspace, normal waits: correct and OK again
    out, ids, wt = _call(fn, w, d, rd, sd, ws)
    assert M.moe_workspace_status(ws) == M.MOE_OK
    ref, rows = ref_fn()
    alt = HP.check_routing(ref, ids, wt, w.k)
    err = HP.rel_l2(out, rows(alt))
    assert err < HP.FP32_TOL, err


@pytest.mark.parametrize("name,w,path", PATHS, ids=[p[0] for p in PATHS])
def test_forced_wait_timeout_shows_in_outputs_and_status(name, w, path):
    d = S.gen_inputs(w, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])

    def ref_fn():
        ref = O.layer(d["x"], d["w_router"], None, d["routed"], d["shared"], w.k)
        return ref, lambda alt: HP.reference_rows(ref, d["routed"], d["shared"], ref["tokens"], alt)

    _forced_then_normal(M.moe_layer_forward, w, d, rd, sd, path, ref_fn)


def _rows_with(ref, routed, tok_fn, alt):
    return np.stack([tok_fn(t, alt[t]) if t in alt else ref["out"][t]
                     for t in range(ref["out"].shape[0])])


def test_forced_wait_timeout_fp8_shared_one_token():
    from oracle import fp8_dense as F
    w = PATHS[0][1]
    d = S.gen_inputs(w, 0)
    b8 = S.gen_fp8_bank(w, 0)
    rd, sd = HP.bank_to_dev(d["routed"]), M.Fp8BankTensors.from_numpy(b8, HP.dev())

    def ref_fn():
        ref = F.layer_fp8_shared(d["x"], d["w_router"], None, d["routed"], b8, w.k)
        tok = lambda t, ids: O.token_out_with(ref["x"], ref["logits"], t, ids, d["routed"],  # noqa
                                              ref["y_shared"][t])
        return ref, lambda alt: _rows_with(ref, d["routed"], tok, alt)

    _forced_then_normal(M.moe_layer_forward_fp8_shared, w, d, rd, sd, PATHS[0][2], ref_fn)


def test_forced_wait_timeout_nvfp4_one_token():
    from oracle import nvfp4 as N
    w = PATHS[0][1]
    d = S.gen_inputs(w, 0)
    rn, sn = S.gen_nvfp4_bank(w, 0), S.gen_nvfp4_bank(w, 0, shared=True)
    rd = M.NvBankTensors.from_numpy(rn, HP.dev())
    sd = M.NvBankTensors.from_numpy(sn, HP.dev())

    def ref_fn():
        ref = N.layer_nvfp4(d["x"], d["w_router"], None, rn, sn, w.k)
        tok = lambda t, ids: N.token_out_with_nvfp4(ref["x"], ref["logits"], t, ids, rn,  # noqa
                                                    ref["y_shared"][t])
        return ref, lambda alt: _rows_with(ref, rn, tok, alt)

    _forced_then_normal(M.moe_layer_forward_nvfp4, w, d, rd, sd, PATHS[0][2], ref_fn)


def test_status_of_calls_without_bounded_waits_is_ok():
    # the many-token path has no in-kernel waits; its status reads OK
    w = S.get("tiny")
    T = 40
    d = S.gen_inputs(w, 0)
    x = S.gen_tokens(w, 3, T=T)
    rd, sd = HP.bank_to_dev(d["routed"]), HP.bank_to_dev(d["shared"])
    ws = M.workspace(T, w.H, w.I, w.E, w.k, HP.dev())
    out = torch.empty((T, w.H), dtype=torch.float32, device=HP.dev())
    M.moe_layer_forward(HP.to_dev(x), HP.to_dev(d["w_router"]), None, rd, sd, w.k, out, ws=ws)
    torch.cuda.synchronize()
    assert M.moe_workspace_status(ws) == M.MOE_OK
    assert np.isfinite(out.cpu().numpy()).all()
