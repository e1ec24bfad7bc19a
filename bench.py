#!/usr/bin/env python3
"""One-GPU benchmark of the routed MXFP4 mixture-of-experts layer.

A step is one moe_layer_forward call: router logits, softmax top-k with
renormalised weights, bucketing, every selected routed expert plus the shared
expert (MXFP4 SwiGLU FFNs) and the fixed-order combine, over one batch of
seeded synthetic input already resident in HBM.

Default workload: single-token decode at the real layer shape (1 token,
hidden 5120, 384 experts top-6 + 1 shared, intermediate 2304). To keep the
256 MB Infinity Cache from serving weights across steps, steps rotate over a
pool of distinct tokens and over several copies of the expert bank and router
at distinct addresses (the cache keys on address, so identical contents at a
new address still miss).

Prints one JSON line. `roofline` covers the expert FFN (the kernel that moves
~97 % of the bytes), timed with HIP events on the launch stream in a loop of
moe_expert_ffn_mxfp4 calls that do exactly the layer's expert work (routed
experts plus the shared expert laid out as expert E of one allocation).
`cpu_baseline` times the fp64 oracle on the host on a bounded token sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s vs peak; prefill MFMA util (1 MI355X)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_16BIT_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="decode",
                    choices=["tiny", "decode", "spec5", "prefill2k_zipf", "prefill16k"])
    ap.add_argument("--copies", type=int, default=None, help="bank copies to rotate over")
    ap.add_argument("--pool", type=int, default=None, help="distinct token batches")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline-loop", action="store_true")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    args = parse()
    if args.gpus != 1:
        log("bench.py measures one GPU: this build has no multi-GPU path (the layer would "
            "shard by expert parallelism; see the design notes). Run with --gpus 1.")
        return 2

    import numpy as np
    import torch

    import mxfp4_routed_expert_softmax_amd as M
    import synthetic as S

    w = S.get(args.config)
    small = w.T <= 16
    K = args.steps if args.steps is not None else (500 if small else (20 if w.T <= 2048 else 6))
    W = args.warmup if args.warmup is not None else (50 if small else 2)
    C = args.copies if args.copies is not None else (4 if small else 1)
    P = args.pool if args.pool is not None else (64 if w.T == 1 else (32 if small else 1))

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    lib = M.lib()

    # ---- inputs, resident in HBM before timing ----------------------------
    t0 = time.time()
    routed_np = S.gen_bank(w, 0)
    shared_np = S.gen_bank(w, 0, shared=True)
    keys = ("gate_up_codes", "gate_up_scales", "down_codes", "down_scales")
    ext = {k: torch.from_numpy(np.concatenate([routed_np[k], shared_np[k]], axis=0)).to(dev)
           for k in keys}
    copies = [ext] + [{k: v.clone() for k, v in ext.items()} for _ in range(C - 1)]
    banks = []
    for c in copies:
        banks.append(dict(
            routed=M.BankTensors(*[c[k][: w.E] for k in keys]),
            shared=M.BankTensors(*[c[k][w.E:] for k in keys]),
            both=M.BankTensors(*[c[k] for k in keys])))
    wr0 = torch.from_numpy(S.gen_router(w, 0).view(np.int16)).to(dev).view(torch.bfloat16)
    wrs = [wr0] + [wr0.clone() for _ in range(C - 1)]
    bias_np = S.gen_zipf_bias(w, 0)
    bias = None if bias_np is None else torch.from_numpy(bias_np).to(dev)
    xs_np = np.stack([S.gen_tokens(w, 0, call=i) for i in range(P)])
    x_pool = torch.from_numpy(xs_np.view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    ws = M.workspace(w.T, w.H, w.I, w.E + 1, w.k + 1, dev)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs resident in {time.time() - t0:.1f}s "
        f"({C} bank copies, {P} token batches)")

    # Pre-marshalled arguments: the timed loop makes one C call per step.
    fwd = lib.moe_layer_forward
    sh = stream.cuda_stream
    ws_n = ws.numel()
    import ctypes
    step_args = []
    for i in range(max(P, C) if P % C == 0 or C % P == 0 else P * C):
        b = banks[i % C]
        step_args.append((x_pool[i % P].data_ptr(), wrs[i % C].data_ptr(),
                          None if bias is None else bias.data_ptr(),
                          ctypes.byref(b["routed"].struct), ctypes.byref(b["shared"].struct),
                          w.T, w.k, out.data_ptr(), ids.data_ptr(), wts.data_ptr(),
                          ws.data_ptr(), ws_n, sh))
    n_args = len(step_args)

    def step(i):
        st = fwd(*step_args[i % n_args])
        if st != 0:
            raise M.MoeError("moe_layer_forward", st, M.status_str(st))

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(K):
        step(W + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / K
    tokens_s = K * w.T / (ms / 1e3)
    log(f"[bench] layer: {ms_step * 1e3:.2f} us/step, {tokens_s:,.0f} tokens/s")

    # Touched experts per call (routed union + shared) for the byte count.
    def expert_bytes():
        n = 3 * w.H * w.I
        return n // 2 + n // 32

    # ---- roofline loop: the expert FFN alone ------------------------------
    roof = None
    if not args.no_roofline_loop:
        R = w.T * w.k
        ffn_args, touched = [], []
        keep = []
        for i in range(n_args):
            xi = x_pool[i % P]
            M.moe_router_topk(xi, wrs[i % C], bias, w.k, ids, wts, None, ws)
            off = torch.empty(w.E + 2, dtype=torch.int32, device=dev)
            rt = torch.empty(R + w.T, dtype=torch.int32, device=dev)
            inv = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
            M.moe_permute(ids, w.E, off[: w.E + 1], rt[:R], inv, ws)
            off[w.E + 1] = R + w.T                       # shared expert = bucket E
            rt[R:] = torch.arange(w.T, dtype=torch.int32, device=dev)
            torch.cuda.synchronize()
            counts = (off[1:] - off[:-1]).cpu().numpy()
            touched.append(int((counts > 0).sum()))
            keep.append((off, rt, inv))
            ffn_args.append((xi.data_ptr(), ctypes.byref(banks[i % C]["both"].struct),
                             off.data_ptr(), rt.data_ptr(), w.T, R + w.T))
        y = torch.empty((R + w.T, w.H), dtype=torch.float32, device=dev)
        ffn = lib.moe_expert_ffn_mxfp4

        def fstep(i):
            a = ffn_args[i % n_args]
            st = ffn(*a, y.data_ptr(), ws.data_ptr(), ws_n, sh)
            if st != 0:
                raise M.MoeError("moe_expert_ffn_mxfp4", st, M.status_str(st))

        for i in range(W):
            fstep(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(K):
            fstep(W + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        f_ms = ev0.elapsed_time(ev1) / K
        mean_touched = float(np.mean([touched[(W + i) % n_args] for i in range(K)]))
        if small:
            by = mean_touched * expert_bytes() + w.T * w.H * 2 + (R + w.T) * w.H * 4
            ach = by / (f_ms / 1e3) / 1e9
            roof = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(ach / HBM_PEAK_GBS, 4), traffic=None)
            log(f"[bench] expert FFN: {f_ms * 1e3:.2f} us/call, {mean_touched:.2f} experts "
                f"touched, {by / 1e6:.1f} MB -> {ach:,.0f} GB/s")
        else:
            fl = (R + w.T) * 2.0 * 3 * w.H * w.I
            ach = fl / (f_ms / 1e3) / 1e12
            roof = dict(bound="mfma", achieved=round(ach, 1), peak=MFMA_16BIT_PEAK_TFLOPS,
                        unit="TFLOP/s", frac=round(ach / MFMA_16BIT_PEAK_TFLOPS, 4),
                        traffic=None)
            log(f"[bench] expert FFN: {f_ms:.3f} ms/call, {fl / 1e12:.3f} TFLOP -> "
                f"{ach:,.1f} TFLOP/s ({mean_touched:.0f} experts touched)")

    # ---- CPU baseline: the fp64 oracle on the host -------------------------
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe as O
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        wr_np = S.gen_router(w, 0)
        n_tok, t_cpu, calls = 0, 0.0, 0
        Tcpu = w.T if w.T <= 16 else 1
        while t_cpu < args.cpu_seconds and calls < P:
            xb = xs_np[calls % P][:Tcpu] if w.T <= 16 else xs_np[0][calls:calls + 1]
            ta = time.perf_counter()
            O.layer(xb, wr_np, bias_np, routed_np, shared_np, w.k)
            t_cpu += time.perf_counter() - ta
            n_tok += xb.shape[0]
            calls += 1
        cpu = dict(value=round(n_tok / t_cpu, 3), unit="tokens/s", cores=int(cores),
                   kind="oracle",
                   sample=f"{calls} layer calls of {Tcpu} token(s) of this workload "
                          f"({n_tok} tokens, {t_cpu:.1f} s, fp64 numpy on the host)")
        log(f"[bench] oracle: {cpu['value']} tokens/s on {cores} threads")

    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x mxfp4 -> fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E,
                   "top_k": w.k, "intermediate": w.I, "shared_experts": 1,
                   "bank_copies": C, "token_batches": P},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
