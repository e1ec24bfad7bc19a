"""Workload shapes and seeded generators for the routed MXFP4 MoE layer.

Shapes follow the DeepSeek-V4.1-Flash layer described on the three pages
(384 routed experts with 6 active plus 1 shared: ai.rs article, table in
"What V4.1 Flash is, in bytes"; experts of 3 x 5120 x 2304 FP4 weights:
FreeToken issue #444, "Architecture delta vs deepseek_v4"; packed E2M1 codes
with one E8M0 scale per 32 weights: same issue, janit's comment, section 2).

Every array is produced from its own keyed PCG64 stream, so any one expert,
token or router matrix can be regenerated alone (the oracle checks single
experts of a 6.7 GiB bank without generating the rest):

    [seed, cfg_id, 0, copy, e, m]  expert e (e == E is the shared expert),
                                   matrix m: 0 gate, 1 up, 2 down.
                                   Codes first (uniform bytes), then scales.
    [seed, cfg_id, 1]              router weight, N(0, router_std)
    [seed, cfg_id, 2, i]           token i, N(0, 1)
    [seed, cfg_id, 2, b, 0]        correlated blocks: base vector of block b
    [seed, cfg_id, 2, b, j + 1]    correlated blocks: noise of token j
    [seed, cfg_id, 3]              popularity ranks for the Zipf logit offset
    [seed, cfg_id, 5, copy, e, m]  NVFP4 expert e (e == E: shared): codes,
                                   then E4M3 scales per 16, then the fp32
                                   matrix scale
    [seed, cfg_id, 4, copy, m]     FP8 shared expert (32 x 32 block scales),
                                   matrix m: 0 gate, 1 up, 2 down. Element
                                   bytes first, then scales.

Floating-point samples are drawn in fp64, rounded to fp32 (round to nearest
even) and then to bf16 (round to nearest even on the fp32 bit pattern). The
result is handed out as uint16 bit patterns; both sides decode the same bits.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic layer call: T tokens through an E-expert top-k layer."""

    name: str
    cfg_id: int
    T: int          # tokens per call
    H: int          # hidden size (K of gate/up, N of down)
    E: int          # routed experts
    k: int          # experts chosen per token
    I: int          # expert intermediate size
    exp_lo: int     # E8M0 exponent range (inclusive), scale byte = 127 + exp
    exp_hi: int
    router_std: float = 0.02
    zipf_s: float | None = None     # per-expert popularity offset on logits
    block: int = 0                  # >0: tokens drawn in correlated blocks
    noise: float = 0.5              # correlated blocks: x = base + noise * n
    shared: int = 1                 # shared experts (always weight 1)
    desc: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        return self.T * self.k


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 0, T=8, H=256, E=16, k=2, I=128, exp_lo=-6, exp_hi=-2,
                 desc="8 tokens, hidden 256, 16 experts top-2 + 1 shared, I=128"),
        Workload("decode", 1, T=1, H=5120, E=384, k=6, I=2304, exp_lo=-8, exp_hi=-4,
                 desc="1 token at the real layer shape, 384 experts top-6 + 1 shared"),
        Workload("spec5", 2, T=5, H=5120, E=384, k=6, I=2304, exp_lo=-8, exp_hi=-4,
                 block=5,
                 desc="5-token verification block, correlated tokens"),
        Workload("prefill2k_zipf", 3, T=2048, H=5120, E=384, k=6, I=2304,
                 exp_lo=-8, exp_hi=-4, zipf_s=1.1,
                 desc="2048-token prefill, Zipf(1.1) expert popularity offset"),
        Workload("prefill16k", 4, T=16384, H=5120, E=384, k=6, I=2304,
                 exp_lo=-8, exp_hi=-4,
                 desc="16384-token prefill, uniform router"),
        # The draft head's MoE: 128 routed experts, blocks of 5. Its hidden
        # and intermediate sizes, top-k and shared expert are taken equal to
        # the main layer's (the pages give only the expert count and call
        # its layers full blocks of the main model).
        Workload("draft128", 5, T=5, H=5120, E=128, k=6, I=2304, exp_lo=-8, exp_hi=-4,
                 block=5,
                 desc="draft-head MoE: 5-token block, 128 experts top-6 + 1 shared"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# bf16 bit patterns
# ---------------------------------------------------------------------------

def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE on the fp32 bits); returns uint16.

    Only finite inputs are expected (normal samples)."""
    f = np.ascontiguousarray(np.asarray(v, dtype=np.float64).astype(np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _normal_bf16(key, n: int, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(key)
    return f64_to_bf16_bits(rng.normal(0.0, std, n))


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------

def _matrix(key, n_rows: int, k_cols: int, exp_lo: int, exp_hi: int):
    """Codes [n_rows][k_cols/2] and scales [n_rows][k_cols/32] of one matrix."""
    if k_cols % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(key)
    codes = rng.integers(0, 256, n_rows * (k_cols // 2), dtype=np.uint8)
    scales = (127 + rng.integers(exp_lo, exp_hi + 1, n_rows * (k_cols // 32))).astype(np.uint8)
    return codes.reshape(n_rows, k_cols // 2), scales.reshape(n_rows, k_cols // 32)


def gen_expert(w: Workload, seed: int, e: int, copy: int = 0) -> dict:
    """The six arrays of expert e (e == w.E is the shared expert).

    gate/up: [I][H/2] codes, [I][H/32] scales; down: [H][I/2], [H][I/32].
    Row-major along the reduction dimension K; byte b of a row holds
    elements 2b (low nibble) and 2b+1 (high nibble)."""
    base = [seed, w.cfg_id, 0, copy, e]
    gc, gs = _matrix(base + [0], w.I, w.H, w.exp_lo, w.exp_hi)
    uc, us = _matrix(base + [1], w.I, w.H, w.exp_lo, w.exp_hi)
    dc, ds = _matrix(base + [2], w.H, w.I, w.exp_lo, w.exp_hi)
    return dict(gate_codes=gc, gate_scales=gs, up_codes=uc, up_scales=us,
                down_codes=dc, down_scales=ds)


def bank_shapes(E: int, H: int, I: int) -> dict:
    return dict(
        gate_up_codes=(E, 2, I, H // 2),
        gate_up_scales=(E, 2, I, H // 32),
        down_codes=(E, H, I // 2),
        down_scales=(E, H, I // 32),
    )


def gen_bank(w: Workload, seed: int, copy: int = 0, shared: bool = False,
             experts=None, threads: int | None = None) -> dict:
    """Bank arrays in the library's layout.

    gate_up_codes  [E][2][I][H/2]   (matrix 0 = gate, 1 = up)
    gate_up_scales [E][2][I][H/32]
    down_codes     [E][H][I/2]
    down_scales    [E][H][I/32]

    shared=True gives the one-expert bank of the shared expert. `experts`
    restricts generation to a subset (other slots stay zero)."""
    E = 1 if shared else w.E
    arrs = {k: np.zeros(s, dtype=np.uint8) for k, s in bank_shapes(E, w.H, w.I).items()}
    ids = [0] if shared else (range(w.E) if experts is None else experts)

    def fill(slot: int) -> None:
        x = gen_expert(w, seed, w.E if shared else slot, copy)
        arrs["gate_up_codes"][slot, 0] = x["gate_codes"]
        arrs["gate_up_codes"][slot, 1] = x["up_codes"]
        arrs["gate_up_scales"][slot, 0] = x["gate_scales"]
        arrs["gate_up_scales"][slot, 1] = x["up_scales"]
        arrs["down_codes"][slot] = x["down_codes"]
        arrs["down_scales"][slot] = x["down_scales"]

    n = threads or _threads()
    if n > 1 and len(ids) > 1:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(fill, ids))
    else:
        for s in ids:
            fill(s)
    arrs.update(E=E, H=w.H, I=w.I)
    return arrs


def _fp8_matrix(key, n_rows: int, k_cols: int, exp_lo: int, exp_hi: int,
                e_lo: int = 5, e_hi: int = 9, all_codes: bool = False):
    """E4M3 element bytes [n][k] drawn field by field (sign uniform, exponent
    field uniform in [e_lo, e_hi], mantissa uniform; 1 in 16 bytes zero), or
    uniform over every finite byte (all_codes); E8M0 scale bytes 127 + exp
    for each 32 x 32 block, exp uniform in [exp_lo, exp_hi]."""
    rng = np.random.default_rng(key)
    n = n_rows * k_cols
    if all_codes:
        b = rng.integers(0, 254, n, dtype=np.int64)
        b = np.where(b >= 0x7F, b + 1, b).astype(np.uint8)     # skip the NaN 0x7F, 0xFF
        b[b == 0xFF] = 0xFE
    else:
        sign = rng.integers(0, 2, n, dtype=np.uint8)
        e = rng.integers(e_lo, e_hi + 1, n, dtype=np.uint8)
        m = rng.integers(0, 8, n, dtype=np.uint8)
        b = (sign << 7) | (e << 3) | m
        b[rng.integers(0, 16, n) == 0] = 0
    s = (127 + rng.integers(exp_lo, exp_hi + 1, (n_rows // 32) * (k_cols // 32))).astype(np.uint8)
    return b.reshape(n_rows, k_cols), s.reshape(n_rows // 32, k_cols // 32)


def gen_fp8_bank(w: Workload, seed: int, copy: int = 0, all_codes: bool = False) -> dict:
    """One-expert FP8 bank (the shared expert in the checkpoint's dense
    format): gate_up_w [1][2][I][H], gate_up_scales [1][2][I/32][H/32],
    down_w [1][H][I], down_scales [1][H/32][I/32]."""
    H, I = w.H, w.I
    g = _fp8_matrix([seed, w.cfg_id, 4, copy, 0], I, H, w.exp_lo, w.exp_hi, all_codes=all_codes)
    u = _fp8_matrix([seed, w.cfg_id, 4, copy, 1], I, H, w.exp_lo, w.exp_hi, all_codes=all_codes)
    d = _fp8_matrix([seed, w.cfg_id, 4, copy, 2], H, I, w.exp_lo, w.exp_hi, all_codes=all_codes)
    return dict(gate_up_w=np.stack([g[0], u[0]])[None], gate_up_scales=np.stack([g[1], u[1]])[None],
                down_w=d[0][None], down_scales=d[1][None], E=1, H=H, I=I)


def _nvfp4_matrix(key, n_rows: int, k_cols: int):
    """Codes [n][k/2] (uniform bytes), E4M3 scale bytes [n][k/16] drawn field
    by field (sign 0, exponent field uniform in [4, 8], mantissa uniform),
    and one fp32 matrix scale 2^-5 * (1 + u), u uniform in [0, 1)."""
    rng = np.random.default_rng(key)
    codes = rng.integers(0, 256, n_rows * k_cols // 2, dtype=np.uint8).reshape(n_rows, k_cols // 2)
    n_s = n_rows * k_cols // 16
    e = rng.integers(4, 9, n_s, dtype=np.uint8)
    m = rng.integers(0, 8, n_s, dtype=np.uint8)
    scales = ((e << 3) | m).astype(np.uint8).reshape(n_rows, k_cols // 16)
    g = np.float32(2.0 ** -5 * (1.0 + rng.random()))
    return codes, scales, g


def gen_nvfp4_bank(w: Workload, seed: int, copy: int = 0, shared: bool = False,
                   experts=None) -> dict:
    """NVFP4 bank: gate_up_codes [E][2][I][H/2], gate_up_scales [E][2][I][H/16]
    (E4M3), down_codes [E][H][I/2], down_scales [E][H][I/16], global_scales
    [E][3] fp32 (gate, up, down). Unlisted experts stay zero."""
    E = 1 if shared else w.E
    H, I = w.H, w.I
    a = dict(gate_up_codes=np.zeros((E, 2, I, H // 2), np.uint8),
             gate_up_scales=np.zeros((E, 2, I, H // 16), np.uint8),
             down_codes=np.zeros((E, H, I // 2), np.uint8),
             down_scales=np.zeros((E, H, I // 16), np.uint8),
             global_scales=np.zeros((E, 3), np.float32))
    ids = [0] if shared else (range(w.E) if experts is None else experts)

    def fill(slot: int) -> None:
        e = w.E if shared else slot
        for m in range(3):
            n, kk = (I, H) if m < 2 else (H, I)
            c, s, g = _nvfp4_matrix([seed, w.cfg_id, 5, copy, e, m], n, kk)
            if m < 2:
                a["gate_up_codes"][slot, m], a["gate_up_scales"][slot, m] = c, s
            else:
                a["down_codes"][slot], a["down_scales"][slot] = c, s
            a["global_scales"][slot, m] = g

    n = _threads()
    if n > 1 and len(ids) > 1:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(fill, ids))
    else:
        for slot in ids:
            fill(slot)
    a.update(E=E, H=H, I=I)
    return a


# ---------------------------------------------------------------------------
# router, tokens, bias
# ---------------------------------------------------------------------------

def gen_router(w: Workload, seed: int) -> np.ndarray:
    """Router weight [E][H] as bf16 bits, N(0, router_std)."""
    return _normal_bf16([seed, w.cfg_id, 1], w.E * w.H, w.router_std).reshape(w.E, w.H)


def gen_tokens(w: Workload, seed: int, call: int = 0, T: int | None = None) -> np.ndarray:
    """Activations [T][H] as bf16 bits for call number `call` of a pool.

    Independent tokens use stream index call*T + t. Correlated blocks use
    block index `call`: x_j = base + noise * n_j, sampled in fp64, then
    rounded once to bf16."""
    T = w.T if T is None else T
    if w.block:
        base = np.random.default_rng([seed, w.cfg_id, 2, call, 0]).normal(0.0, 1.0, w.H)
        rows = []
        for j in range(T):
            n = np.random.default_rng([seed, w.cfg_id, 2, call, j + 1]).normal(0.0, 1.0, w.H)
            rows.append(f64_to_bf16_bits(base + w.noise * n))
        return np.stack(rows)
    out = np.empty((T, w.H), dtype=np.uint16)

    def fill(t: int) -> None:
        out[t] = _normal_bf16([seed, w.cfg_id, 2, call * T + t], w.H)

    if T > 256:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(T)))
    else:
        for t in range(T):
            fill(t)
    return out


def gen_zipf_bias(w: Workload, seed: int) -> np.ndarray | None:
    """Per-expert logit offset -s*ln(rank) with a seeded rank permutation.

    Adding ln of a Zipf(s) popularity to a logit multiplies that expert's
    softmax numerator by rank^-s. Returned as fp32 (both sides consume these
    exact fp32 values), or None when the workload has no offset."""
    if w.zipf_s is None:
        return None
    rank = np.random.default_rng([seed, w.cfg_id, 3]).permutation(w.E) + 1
    return (-w.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


def gen_inputs(w: Workload, seed: int = 0, call: int = 0, copy: int = 0,
               with_bank: bool = True) -> dict:
    """Everything one layer call consumes."""
    d = dict(workload=w, seed=seed,
             x=gen_tokens(w, seed, call),
             w_router=gen_router(w, seed),
             bias=gen_zipf_bias(w, seed))
    if with_bank:
        d["routed"] = gen_bank(w, seed, copy)
        d["shared"] = gen_bank(w, seed, copy, shared=True)
    return d

