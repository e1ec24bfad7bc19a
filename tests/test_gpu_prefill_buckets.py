"""Whole buckets of the grouped GEMM at the real layer shape.

moe_expert_ffn_mxfp4 runs the MFMA grouped GEMM above 128 rows. Here it runs
on the real routing of the 2k-token Zipf workload and of the 16k-token
uniform workload (offsets and row order from the oracle's own bucketing of
those tokens), over a 384-expert bank in which only the buckets under test
hold weights. So the GEMM plans its tiles for the real bucket sizes at
E = 384 (the 64-workgroup plan, the per-XCD stretches), and every row of the
chosen buckets is compared with the fp64 oracle:

  * the largest 2k-token bucket (about 1,600 rows: a dozen row blocks);
  * buckets of 1, 2 and 3 rows (a 128-row tile nearly all padding);
  * a bucket of 129..255 rows (a full block and a ragged one);
  * four full 16k-token buckets (about 256 rows each);
  * the shared expert as a one-expert bucket of 1,000 rows, whose last row
    block is ragged (1,000 = 7 x 128 + 104).

Rows of the experts that hold no weights must come out exactly zero. The
tolerance is the GEMM path's (h carried in fp16): GEMM_TOL over each bucket,
and at most 4 x GEMM_TOL on any single row.
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
    torch.cuda.synchronize()


def _launches():
    return [M.moe_launch_name(i) for i in range(M.moe_last_call_launches())]


def _run_ffn(x_bits, bank, offsets, row_token, R):
    T = x_bits.shape[0]
    bd = HP.bank_to_dev(bank)
    y = torch.full((R, bank["H"]), float("nan"), dtype=torch.float32, device=HP.dev())
    ws = M.workspace(T, bank["H"], bank["I"], bank["E"], max(1, -(-R // T)), HP.dev())
    off = None if offsets is None else HP.to_dev(offsets.astype(np.int32))
    rt = None if row_token is None else HP.to_dev(row_token.astype(np.int32))
    M.moe_expert_ffn_mxfp4(HP.to_dev(x_bits), bd, off, rt, R, y, ws)
    torch.cuda.synchronize()
    names = _launches()
    assert "gemm_gateup_kernel" in names and "gemm_down_kernel" in names, names
    return y.cpu().numpy().astype(np.float64)


def _compare_rows(got, ref, label):
    err = HP.rel_l2(got, ref)
    row = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    print(f"{label}: {got.shape[0]} rows, rel-L2 {err:.3e}, worst row {row.max():.3e}", flush=True)
    assert np.isfinite(got).all(), label
    assert err <= HP.GEMM_TOL, (label, err)
    assert row.max() <= 4 * HP.GEMM_TOL, (label, row.max())


def _bucket_case(name, pick):
    w = S.get(name)
    x = S.gen_tokens(w, 0)
    r = O.route(x, S.gen_router(w, 0), S.gen_zipf_bias(w, 0), w.k)
    off, rt = r["offsets"], r["row_token"]
    counts = np.diff(off)
    chosen = pick(counts)
    bank = S.gen_bank(w, 0, experts=chosen)
    R = w.T * w.k
    print(f"{name}: buckets {[(int(e), int(counts[e])) for e in chosen]}", flush=True)
    y = _run_ffn(x, bank, off, rt, R)
    xf = O.bf16_to_f64(x)
    for e in chosen:
        rows = np.arange(off[e], off[e + 1])
        wg, wu, wd = O.expert_weights(bank, int(e))
        ref = O.expert_ffn(xf[rt[rows]], wg, wu, wd)
        _compare_rows(y[rows], ref, f"{name} expert {e} ({rows.size} rows)")
    others = np.ones(R, bool)
    for e in chosen:
        others[off[e]:off[e + 1]] = False
    assert np.array_equal(y[others], np.zeros_like(y[others])), "rows of empty experts"


def test_gemm_real_shape_prefill2k_largest_small_and_ragged_buckets():
    def pick(counts):
        order = np.argsort(-counts, kind="stable")
        chosen = [int(order[0])]
        for c in (1, 2, 3):
            hit = np.flatnonzero(counts == c)
            if hit.size:
                chosen.append(int(hit[0]))
        rag = np.flatnonzero((counts > 128) & (counts < 256))
        if rag.size:
            chosen.append(int(rag[0]))
        assert counts[chosen[0]] > 1000 and len(chosen) >= 4, counts[chosen]
        return sorted(chosen)

    _bucket_case("prefill2k_zipf", pick)


def test_gemm_real_shape_prefill16k_full_buckets():
    def pick(counts):
        order = np.argsort(counts, kind="stable")
        n = counts.size
        return sorted(int(e) for e in (order[0], order[n // 3], order[2 * n // 3], order[-1]))

    _bucket_case("prefill16k", pick)


def test_gemm_real_shape_shared_bucket_ragged_last_block():
    w = S.get("prefill2k_zipf")
    T = 1000                                  # 7 row blocks of 128 and one of 104
    x = S.gen_tokens(w, 0)[:T]
    shared = S.gen_bank(w, 0, shared=True)
    y = _run_ffn(x, shared, None, None, T)
    ref = O.expert_ffn(O.bf16_to_f64(x), *O.expert_weights(shared, 0))
    _compare_rows(y, ref, "shared expert, 1000 rows")
