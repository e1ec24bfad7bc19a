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

Prints one JSON line. `roofline` covers the layer's dominant kernel: a
second loop of the same calls sets the library's timing hook, which attaches
HIP start / stop events to every kernel launch, and the kernel with the
largest mean duration is reported against its algorithmic bytes (HBM-bound)
or flops (MFMA-bound) per launch. `cpu_baseline` times the fp64 oracle on the
host on a bounded token sample.
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
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (the rate of fp8 x fp4 scaled MFMA)
# kernels whose MFMA peak is not the 16-bit one
MFMA_PEAK_OF = {"gemm_mx_gateup_kernel": MFMA_FP8_PEAK_TFLOPS,
                "gemm_mx_down_kernel": MFMA_FP8_PEAK_TFLOPS}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="decode",
                    choices=["tiny", "decode", "spec5", "prefill2k_zipf", "prefill16k",
                             "draft128"])
    ap.add_argument("--copies", type=int, default=None, help="bank copies to rotate over")
    ap.add_argument("--pool", type=int, default=None, help="distinct token batches")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline-loop", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="default decode run only: skip the 16k-token prefill sub-record")
    ap.add_argument("--verify-sweep", action="store_true",
                    help="instead of one workload: verification blocks of 2..8 correlated "
                         "tokens at the decode shape; per block size, time, the union of "
                         "routed experts and the bytes it costs")
    ap.add_argument("--mxfp8-act", action="store_true",
                    help="time moe_layer_forward_mxfp8_act, the opt-in mode with MXFP8 "
                         "activations on the scaled fp8 x fp4 MFMA (an approximation of the "
                         "layer; its error against the exact layer is reported)")
    ap.add_argument("--fp8-shared", action="store_true",
                    help="time moe_layer_forward_fp8_shared: the shared expert in the "
                         "checkpoint's FP8 format (E4M3, 32 x 32 ue8m0 block scales)")
    ap.add_argument("--nvfp4", action="store_true",
                    help="time moe_layer_forward_nvfp4: routed and shared experts in NVFP4 "
                         "(E2M1 codes, E4M3 scale per 16, fp32 matrix scale)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 3 plain device copies of BYTES bytes (the reference "
                         "reading for the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_info():
    """The host the CPU baseline runs on: CPU model, numpy's BLAS and the
    cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name')} {b.get('version', '')}".strip()
    except Exception:
        pass
    try:
        from threadpoolctl import threadpool_info
        rt = [f"{i.get('internal_api')} ({i.get('num_threads')} threads)" for i in threadpool_info()
              if i.get("user_api") == "blas"]
        if rt:
            blas = f"{blas}; runtime {', '.join(rt)}"
    except Exception:
        pass
    return dict(cpu_model=model, blas=blas, affinity_cores=len(os.sched_getaffinity(0)))


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def main() -> int:
    args = parse()
    if args.gpus != 1:
        log("bench.py measures one GPU: there is no multi-GPU path (the layer would "
            "shard by expert parallelism). Run with --gpus 1.")
        return 2

    import numpy as np
    import torch

    import mxfp4_routed_expert_softmax_amd as M
    import synthetic as S

    if args.copy_probe:
        n = args.copy_probe
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return 0

    if args.verify_sweep:
        return verify_sweep(args, M, S, np, torch)

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
    if sum([args.nvfp4, args.fp8_shared, args.mxfp8_act]) > 1:
        log("--nvfp4, --fp8-shared and --mxfp8-act are separate modes")
        return 2
    gen = S.gen_nvfp4_bank if args.nvfp4 else S.gen_bank
    routed_np = gen(w, 0)
    shared_np = gen(w, 0, shared=True)
    keys = ("gate_up_codes", "gate_up_scales", "down_codes", "down_scales") + \
        (("global_scales",) if args.nvfp4 else ())
    ext = {k: torch.from_numpy(np.concatenate([routed_np[k], shared_np[k]], axis=0)).to(dev)
           for k in keys}
    copies = [ext] + [{k: v.clone() for k, v in ext.items()} for _ in range(C - 1)]
    banks = []
    BT = M.NvBankTensors if args.nvfp4 else M.BankTensors
    for c in copies:
        banks.append(dict(
            routed=BT(*[c[k][: w.E] for k in keys]),
            shared=BT(*[c[k][w.E:] for k in keys])))
    if args.fp8_shared:
        if args.mxfp8_act:
            log("--fp8-shared and --mxfp8-act are separate modes")
            return 2
        shared8_np = S.gen_fp8_bank(w, 0)
        s8 = M.Fp8BankTensors.from_numpy(shared8_np, dev)
        for i, b in enumerate(banks):
            b["shared"] = s8 if i == 0 else M.Fp8BankTensors(*[t.clone() for t in s8.tensors])
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
    fwd_name = ("moe_layer_forward_mxfp8_act" if args.mxfp8_act else
                "moe_layer_forward_fp8_shared" if args.fp8_shared else
                "moe_layer_forward_nvfp4" if args.nvfp4 else "moe_layer_forward")
    fwd = getattr(lib, fwd_name)
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
            raise M.MoeError(fwd_name, st, M.status_str(st))

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

    # ---- expert load of the last batch (rows per expert) ------------------
    load = None
    if w.T > 16:
        cnt = torch.bincount(ids.reshape(-1).long(), minlength=w.E).cpu().numpy()
        act = cnt[cnt > 0]
        load = dict(active_experts=int(act.size), rows=int(cnt.sum()),
                    rows_per_active_expert=dict(
                        mean=round(float(act.mean()), 1), max=int(act.max()),
                        p50=int(np.percentile(act, 50)), p90=int(np.percentile(act, 90)),
                        p99=int(np.percentile(act, 99))),
                    rows_in_top_10pct_experts=round(float(np.sort(act)[::-1][: max(1, act.size // 10)].sum()
                                                          / cnt.sum()), 3))
        log(f"[bench] expert load: {load}")

    # distinct routed experts of each token batch (the routing is the same
    # for every bank copy)
    U = []
    for p in range(P):
        M.moe_router_topk(x_pool[p], wrs[0], bias, w.k, ids, wts, None, ws)
        U.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()
    layer_roof = layer_roofline(w, U, W, K, P, ms_step, args)
    log(f"[bench] layer roofline: {layer_roof}")

    # ---- roofline: the dominant kernel, timed with HIP events --------------
    # A second loop makes the same calls as the timed one with the library's
    # timing hook set: every kernel launch then carries a start and a stop
    # event that the runtime stamps at that kernel's dispatch begin and end
    # on the launch stream. The kernel with the largest mean duration is the
    # one reported, against its algorithmic bytes (HBM-bound kernels) or
    # flops (MFMA-bound kernels) per launch.
    roof = None
    if not args.no_roofline_loop:
        roof = kernel_roofline(args, w, M, lib, torch, np, step, U, P, W, K,
                               shared8=args.fp8_shared)
    # ---- CPU baseline: the fp64 oracle on the host -------------------------
    cpu = None
    mx_err = None
    if args.mxfp8_act:
        # error of the mode against the exact layer on a few tokens of the
        # last timed batch (the oracle's own rounding reproduces the mode)
        from oracle import moe as O
        from oracle import mxfp8_act as MXO
        step(W + K - 1)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        xb = xs_np[(W + K - 1) % P]
        tok = sorted(set([0, w.T // 3, w.T // 2, w.T - 1]))
        ex = O.layer(xb, S.gen_router(w, 0), bias_np, routed_np, shared_np, w.k, tokens=tok)["out"]
        mx = MXO.layer_mx(xb, S.gen_router(w, 0), bias_np, routed_np, shared_np, w.k,
                          tokens=tok)["out"]
        rel = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))
        mx_err = dict(tokens=tok, rel_l2_vs_exact_layer=round(rel(got[tok], ex), 5),
                      rel_l2_vs_mode_oracle=round(rel(got[tok], mx), 6))
        log(f"[bench] mxfp8-act error on tokens {tok}: {mx_err}")
    if not args.no_cpu_baseline:
        from oracle import moe as O
        from oracle import mxfp8_act as MXO
        layer_fn = MXO.layer_mx if args.mxfp8_act else O.layer
        if args.fp8_shared:
            from oracle import fp8_dense as F8O
            layer_fn = F8O.layer_fp8_shared
            shared_np = shared8_np
        if args.nvfp4:
            from oracle import nvfp4 as NVO
            layer_fn = NVO.layer_nvfp4
        cores = cpu_threads()
        wr_np = S.gen_router(w, 0)
        n_tok, t_cpu, calls = 0, 0.0, 0
        Tcpu = w.T if w.T <= 16 else 1
        while t_cpu < args.cpu_seconds and calls < (P if w.T <= 16 else w.T):
            xb = xs_np[calls % P][:Tcpu] if w.T <= 16 else xs_np[0][calls:calls + 1]
            ta = time.perf_counter()
            layer_fn(xb, wr_np, bias_np, routed_np, shared_np, w.k)
            t_cpu += time.perf_counter() - ta
            n_tok += xb.shape[0]
            calls += 1
        cpu = dict(value=round(n_tok / t_cpu, 3), unit="tokens/s", cores=int(cores),
                   kind="oracle",
                   sample=f"{calls} layer calls of {Tcpu} token(s) of this workload "
                          f"({n_tok} tokens, {t_cpu:.1f} s, fp64 numpy on the host)",
                   **host_info())
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
        "dtype": ("mxfp8 x mxfp4 -> fp32" if args.mxfp8_act else
                  "bf16 x nvfp4 -> fp32" if args.nvfp4 else
                  "bf16 x mxfp4 (shared: bf16 x fp8) -> fp32" if args.fp8_shared else
                  "bf16 x mxfp4 -> fp32"),
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E,
                   "top_k": w.k, "intermediate": w.I, "shared_experts": 1,
                   "bank_copies": C, "token_batches": P,
                   "expert_activations": "mxfp8" if args.mxfp8_act else "bf16/fp16/fp32",
                   "expert_format": "nvfp4" if args.nvfp4 else "mxfp4",
                   "shared_expert_format": "fp8 e4m3, 32x32 ue8m0 blocks" if args.fp8_shared
                   else "nvfp4" if args.nvfp4 else "mxfp4"},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "cpu_baseline": cpu,
    }
    if (w.name == "decode" and not (args.nvfp4 or args.fp8_shared or args.mxfp8_act)
            and not args.no_prefill):
        del x_pool, ws
        line["prefill16k"] = prefill_record(args, M, S, np, torch, banks[0], routed_np, shared_np)
    if mx_err is not None:
        line["mxfp8_act_error"] = mx_err
    if load is not None:
        line["expert_load"] = load
    print(json.dumps(line), flush=True)
    return 0



def prefill_record(args, M, S, np, torch, bank, routed_np, shared_np):
    """The prefill half of the metric beside the decode line: 16384 tokens of
    the 16k-token workload (its seeded tokens and uniform bf16 router) through
    the same layer, whose experts are the decode run's bank copy 0 (the same
    shape and recipe; the expert values do not change the work). Layer time,
    the event-timed grouped GEMMs against the 16-bit MFMA peak, the layer's
    roofline, and the fp64 oracle on a bounded sample of tokens, which also
    gives the GPU's error on those tokens."""
    from oracle import moe as O
    w = S.get("prefill16k")
    dev = torch.device("cuda:0")
    t0 = time.time()
    x_np = S.gen_tokens(w, 0)
    wr_np = S.gen_router(w, 0)
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    wr = torch.from_numpy(wr_np.view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    ws = M.workspace(w.T, w.H, w.I, w.E, w.k, dev)
    torch.cuda.synchronize()
    log(f"[bench] prefill16k: inputs resident in {time.time() - t0:.1f}s")

    def call(i):
        M.moe_layer_forward(x, wr, None, bank["routed"], bank["shared"], w.k, out, ids, wts, ws)

    Wp, Kp = 2, 5
    for i in range(Wp):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(Kp):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / Kp
    U = int(torch.unique(ids).numel())
    kern = sweep_kernel_times(M, torch, np, call, Kp)
    gemms = {}
    for name in ("gemm_gateup_kernel", "gemm_down_kernel", "gemm_down_combine_kernel"):
        if name in kern:
            fl = kernel_work(name, w, U)[1][0]
            tf = fl / (kern[name] * 1e-6) / 1e12
            gemms[name] = dict(us=kern[name], tflop=round(fl / 1e12, 3), tflops=round(tf, 1),
                               mfma_frac=round(tf / MFMA_16BIT_PEAK_TFLOPS, 4))
    layer = layer_roofline(w, [U], 0, 1, 1, ms, args)
    rec = dict(workload="prefill16k", tokens=w.T, steps=Kp, warmup=Wp, ms_per_step=round(ms, 4),
               tokens_per_s=round(w.T / (ms / 1e3), 1), active_experts=U,
               bank="the decode run's bank copy 0 (same shape and recipe)",
               layer_roofline=layer, gemm=gemms, kernels_us=kern)
    log(f"[bench] prefill16k: {ms:.3f} ms/step, {rec['tokens_per_s']:,.0f} tokens/s; {gemms}")
    if not args.no_cpu_baseline:
        ids_np = ids.cpu().numpy()
        got = out.cpu().numpy()
        budget, t_cpu, toks, errs = 10.0, 0.0, [], []
        rng = np.random.default_rng(7)
        for t in rng.permutation(w.T):
            if t_cpu >= budget or len(toks) >= 64:
                break
            ta = time.perf_counter()
            r = O.layer(x_np[t:t + 1], wr_np, None, routed_np, shared_np, w.k)
            t_cpu += time.perf_counter() - ta
            toks.append(int(t))
            if r["margin"][0] > 1e-4 and set(r["ids"][0].tolist()) == set(ids_np[t].tolist()):
                errs.append((got[t], r["out"][0]))
        rel = (float(np.linalg.norm(np.stack([a - b for a, b in errs]))
                     / np.linalg.norm(np.stack([b for _, b in errs]))) if errs else None)
        rec["cpu_baseline"] = dict(
            value=round(len(toks) / t_cpu, 3), unit="tokens/s", cores=int(cpu_threads()),
            kind="oracle",
            sample=f"{len(toks)} single-token oracle calls on tokens drawn from the 16384 "
                   f"({t_cpu:.1f} s, fp64 numpy on the host)", **host_info())
        rec["rel_l2_vs_oracle_on_sample"] = None if rel is None else round(rel, 7)
        log(f"[bench] prefill16k oracle: {rec['cpu_baseline']['value']} tokens/s; "
            f"GPU rel-L2 on {len(errs)} sampled tokens {rel}")
    return rec


def sweep_kernel_times(M, torch, np, call, n):
    """Mean duration (us) of each kernel of `call` over n calls, from events the
    library records at each launch's dispatch begin and end."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    call(0)
    torch.cuda.synchronize()
    nl = M.moe_last_call_launches()
    names = [M.moe_launch_name(i) for i in range(nl)]
    evs = []
    for _ in range(n):
        arr = (ctypes.c_void_p * (2 * nl))()
        for j in range(2 * nl):
            e = ctypes.c_void_p()
            hip.hipEventCreate(ctypes.byref(e))
            arr[j] = e.value
        evs.append(arr)
    try:
        for i in range(n):
            M.moe_set_kernel_events(evs[i], nl)
            call(i)
        M.moe_set_kernel_events(None, 0)
        torch.cuda.synchronize()
        f = ctypes.c_float()
        dur = np.zeros((n, nl))
        for i in range(n):
            for j in range(nl):
                hip.hipEventElapsedTime(ctypes.byref(f), evs[i][2 * j], evs[i][2 * j + 1])
                dur[i, j] = f.value * 1e3
    finally:
        M.moe_set_kernel_events(None, 0)
        for arr in evs:
            for e in arr:
                hip.hipEventDestroy(e)
    return {nm: round(float(d), 2) for nm, d in zip(names, dur.mean(axis=0))}


def verify_sweep(args, M, S, np, torch):
    """A verification block of K+1 tokens pays for the union of its tokens'
    experts (ai.rs article, "The draft head that works and does not pay").
    For K+1 = 2..8 correlated tokens (block recipe of spec5) at the decode
    shape: time per block, the mean union |U| of routed experts, and the
    expert bytes (|U| + 1 shared) x 18.8 MB it reads."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = S.get("spec5")
    K = args.steps if args.steps is not None else 200
    W = args.warmup if args.warmup is not None else 20
    C, P = 4, 16
    routed_np = S.gen_bank(base, 0)
    shared_np = S.gen_bank(base, 0, shared=True)
    keys = ("gate_up_codes", "gate_up_scales", "down_codes", "down_scales")
    banks = []
    for c in range(C):
        banks.append((M.BankTensors(*[torch.from_numpy(routed_np[k]).to(dev) for k in keys]),
                      M.BankTensors(*[torch.from_numpy(shared_np[k]).to(dev) for k in keys])))
    del routed_np, shared_np
    wr = torch.from_numpy(S.gen_router(base, 0).view(np.int16)).to(dev).view(torch.bfloat16)
    expert_bytes = 3 * base.I * base.H * 17 // 32
    rows = []
    for T in range(2, 9):
        w = S.Workload(f"verify{T}", base.cfg_id, T=T, H=base.H, E=base.E, k=base.k, I=base.I,
                       exp_lo=base.exp_lo, exp_hi=base.exp_hi, block=T, noise=base.noise)
        xs = [torch.from_numpy(S.gen_tokens(w, 0, call=i).view(np.int16)).to(dev)
              .view(torch.bfloat16) for i in range(P)]
        out = torch.empty((T, w.H), dtype=torch.float32, device=dev)
        ids = torch.empty((T, w.k), dtype=torch.int32, device=dev)
        wts = torch.empty((T, w.k), dtype=torch.float32, device=dev)
        ws = M.workspace(T, w.H, w.I, w.E + 1, w.k + 1, dev)
        U = []
        for x in xs:
            M.moe_router_topk(x, wr, None, w.k, ids, wts, None, ws)
            U.append(int(torch.unique(ids).numel()))
        for i in range(W):
            rd, sd = banks[i % C]
            M.moe_layer_forward(xs[i % P], wr, None, rd, sd, w.k, out, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            rd, sd = banks[i % C]
            M.moe_layer_forward(xs[i % P], wr, None, rd, sd, w.k, out, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        per_kernel = sweep_kernel_times(M, torch, np, lambda i: M.moe_layer_forward(
            xs[i % P], wr, None, banks[i % C][0], banks[i % C][1], w.k, out, ws=ws), 50)
        u = float(np.mean(U))
        union = (u + 1) * expert_bytes
        path = [M.moe_launch_name(i) for i in range(M.moe_last_call_launches())]
        row = dict(tokens=T, us_per_block=round(us, 2), tokens_per_s=round(T / us * 1e6, 1),
                   union_routed_experts=round(u, 2), union_bytes=int(union),
                   bytes_per_token=int(union / T), union_gbs=round(union / us / 1e3, 1),
                   launches=path, kernel_us=per_kernel)
        rows.append(row)
        log(f"[sweep] T={T}: {us:8.2f} us/block, {T / us * 1e6:9,.0f} tokens/s, |U| = {u:5.2f}, "
            f"{union / 1e6:7.1f} MB union ({union / T / 1e6:6.1f} MB/token) -> "
            f"{union / us / 1e3:6.0f} GB/s; "
            + ", ".join(f"{k} {v:.1f}" for k, v in per_kernel.items()))
        del ws
    print(json.dumps({"verify_sweep": rows, "decode_shape": {"H": base.H, "E": base.E, "k": base.k,
                                                             "I": base.I, "shared_experts": 1},
                      "block_recipe": "x_t = bf16(b + 0.5 n_t), b, n_t ~ N(0,1)^H",
                      "steps": K, "warmup": W, "bank_copies": C, "token_batches": P}), flush=True)
    return 0


# Algorithmic work per launch of each kernel, from the call's shape and the
# number U of distinct routed experts it touched. Bytes count every array a
# kernel must read or write once (weights at 17/32 byte per weight: codes plus
# one E8M0 byte per 32); flops count 2 per multiply-add of the expert FFN.
def kernel_work(name, w, U, shared=True, nvfp4=False, shared8=False):
    H, I, T, R = w.H, w.I, w.T, w.T * w.k
    if name == "gateup_fused_kernel" and shared8:
        # one token with the FP8 shared expert streamed in the same launch:
        # the MXFP4 routed work plus the FP8 expert (1 byte per weight, 1 per
        # 32 x 32 block), its h and y rows written and read back
        _, b = kernel_work(name, w, U, False)
        return "hbm", b + 3 * H * I + 3 * (H // 32) * (I // 32) + T * I * 8 + T * H * 8
    if name == "fp8_gateup_gemv_kernel":
        # the FP8 shared expert's gate/up: 1 byte per weight, 1 per 32 x 32 block
        return "hbm", 2 * I * H + 2 * (I // 32) * (H // 32) + T * H * 2 + T * I * 4
    if name == "fp8_down_gemv_kernel":
        return "hbm", H * I + (H // 32) * (I // 32) + T * I * 4 + T * H * 4
    if name == "gemm_fp8w_gateup_kernel":
        return "gemm", (T * 2.0 * 2 * H * I, 2 * I * H + T * H * 2 + T * I * 2)
    if name == "gemm_fp8w_down_kernel":
        return "gemm", (T * 2.0 * H * I, H * I + T * I * 2 + T * H * 4)
    # gate + up and down of one expert: MXFP4 17/32 byte per weight, NVFP4
    # 9/16 (a scale byte per 16) plus its fp32 matrix scales
    gu_expert = 2 * I * H * 9 // 16 + 8 if nvfp4 else 2 * I * H * 17 // 32
    dn_expert = I * H * 9 // 16 + 4 if nvfp4 else I * H * 17 // 32
    if name == "gateup_gemv_kernel":
        # bucketed rows: the U experts' (+ shared) gate/up read once per 4 rows
        return "hbm", (U + (1 if shared else 0)) * gu_expert + (R + (T if shared else 0)) * (H * 2 + I * 4)
    if name == "down_gemv_kernel":
        return "hbm", (U + (1 if shared else 0)) * dn_expert + (R + (T if shared else 0)) * (I * 4 + H * 4)
    if name == "gateup_fused_kernel":
        # the whole one-token layer: router rows, routing, gate/up and down of
        # the routed experts and the shared one, each h row and y row written
        # and read back once, the output row and the k ids and weights
        rows = R + (T if shared else 0)
        return "hbm", w.E * H * 2 + T * H * 2 + T * w.E * 4 \
            + (U + (1 if shared else 0)) * (gu_expert + dn_expert) \
            + rows * (I * 8 + H * 8) + T * H * 4 + T * w.k * 8
    if name == "route_block_kernel":
        # block of tokens: router rows, the routing, the shared expert's
        # gate/up for every token of the block
        b = w.E * H * 2 + T * H * 2 + T * w.E * 4
        if shared:
            b += gu_expert + T * I * 4
        if shared8:
            # the FP8 shared expert's gate/up: 1 byte per weight, 1 per block
            b += 2 * I * H + 2 * (I // 32) * (H // 32) + T * I * 4
        return "hbm", b
    if name == "gateup_block_kernel":
        # gate/up of the U routed experts, each read once for all the block's
        # tokens routed to it, h rows written; then the shared expert's down
        # rows for every token
        b = U * gu_expert + T * H * 2 + R * I * 4
        if shared:
            b += dn_expert + T * I * 4 + T * H * 4
        if shared8:
            b += H * I + (H // 32) * (I // 32) + T * I * 4 + T * H * 4
        return "hbm", b
    if name in ("down_block_kernel", "down_block_mfma_kernel"):
        # down of the U routed experts, h rows read, y rows written as value
        # words and read back by the launch's combine workgroups, with the
        # shared rows; the output rows and the k ids and weights
        sh_rows = T if shared or shared8 else 0
        return "hbm", U * dn_expert + R * I * 4 + R * H * 16 + sh_rows * H * 4 + T * H * 4 \
            + T * w.k * 8
    if name in ("gateup_stream_kernel", "gateup_kernel"):
        # routed gate/up of the U experts (+ the shared expert's down rows)
        b = U * gu_expert + T * H * 2 + R * I * 4
        if shared:
            b += dn_expert + T * I * 4 + T * H * 4
        return "hbm", b
    if name == "down_kernel":
        # routed down of the U experts, then the combine
        return "hbm", U * dn_expert + R * I * 4 + R * H * 4 + (T * H * 4 if shared else 0) \
            + T * H * 4 + T * w.k * 8
    if name == "route_kernel":
        # router GEMV, top-k, bucketing (+ the shared expert's gate/up)
        b = w.E * w.H * 2 + T * H * 2 + T * w.E * 4
        if shared:
            b += gu_expert + T * I * 4
        return "hbm", b
    rows = R + (T if shared else 0)
    # grouped GEMMs: the flops, and the bytes they cannot avoid (each touched
    # expert's weights once, the activations once, the outputs once); the
    # bound is whichever takes longer at its peak
    if name == "gemm_gateup_kernel":
        return "gemm", (rows * 2.0 * 2 * H * I,
                        (U + (1 if shared else 0)) * gu_expert + T * H * 2 + rows * I * 2)
    if name == "gemm_down_kernel":
        # with an MXFP4 or NVFP4 shared expert the layer runs its down tiles
        # in gemm_down_combine_kernel: this launch takes the routed rows
        return "gemm", (R * 2.0 * H * I, U * dn_expert + R * I * 2 + R * H * 4)
    if name == "gemm_down_combine_kernel":
        # the shared expert's down rows, each token combined in the epilogue:
        # the k routed y rows read, the output written
        return "gemm", (T * 2.0 * H * I, dn_expert + T * I * 2 + R * H * 4 + T * H * 4)
    if name == "gemm_mx_gateup_kernel":
        # activations and h at one byte plus one scale byte per 32
        return "gemm", (rows * 2.0 * 2 * H * I,
                        (U + (1 if shared else 0)) * gu_expert + T * H * 33 // 32
                        + rows * I * 33 // 32)
    if name == "gemm_mx_down_kernel":
        return "gemm", (rows * 2.0 * H * I,
                        (U + (1 if shared else 0)) * dn_expert + rows * I * 33 // 32
                        + rows * H * 4)
    if name == "quant_mxfp8_kernel":
        return "hbm", T * H * 2 + T * H * 33 // 32
    if name in ("router_mfma_kernel", "router_mfma_lds_kernel"):
        return "mfma", T * 2.0 * w.E * H
    return None, None


def expert_bytes(w, fmt):
    """Weight bytes of one expert (gate, up and down) in a bank format."""
    n = 3 * w.H * w.I
    if fmt == "nvfp4":
        return n // 2 + n // 16 + 12
    if fmt == "fp8":
        return n + 3 * (w.H // 32) * (w.I // 32)
    return n // 2 + n // 32


def layer_roofline(w, U, W, K, P, ms_step, args):
    """The whole layer call against its roofline. Few tokens: HBM-bound,
    on the selected experts' weight bytes (the union of the routed experts
    the call touched, plus the shared expert) per call; this is the decode
    model of bandwidth over routed expert bytes per token. Many tokens: the
    layer's flops (router + routed and shared experts, 2 per multiply-add)
    against the MFMA peak, with the HBM fraction of the touched experts'
    weights beside it."""
    import numpy as np
    routed_fmt = "nvfp4" if args.nvfp4 else "mxfp4"
    shared_fmt = "fp8" if args.fp8_shared else routed_fmt
    u = float(np.mean([U[(W + i) % P] for i in range(K)]))
    by = u * expert_bytes(w, routed_fmt) + expert_bytes(w, shared_fmt)
    t = ms_step / 1e3
    hbm = by / t / 1e9
    if w.T <= 16:
        return dict(bound="hbm", basis="selected experts' weight bytes (routed union + shared) "
                    "per layer call / ms_per_step", experts=round(u + 1, 2), bytes=int(by),
                    achieved=round(hbm, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(hbm / HBM_PEAK_GBS, 4))
    fl = w.T * (2.0 * w.E * w.H + (w.k + 1) * 6.0 * w.H * w.I)
    mpeak = MFMA_FP8_PEAK_TFLOPS if args.mxfp8_act else MFMA_16BIT_PEAK_TFLOPS
    tf = fl / t / 1e12
    bound = "mfma" if fl / (mpeak * 1e12) >= by / (HBM_PEAK_GBS * 1e9) else "hbm"
    return dict(bound=bound, basis="layer flops (router + routed and shared experts) and the "
                "touched experts' weight bytes per layer call / ms_per_step",
                flops=fl, bytes=int(by),
                achieved=round(tf, 1) if bound == "mfma" else round(hbm, 1),
                peak=mpeak if bound == "mfma" else HBM_PEAK_GBS,
                unit="TFLOP/s" if bound == "mfma" else "GB/s",
                frac=round((tf / mpeak) if bound == "mfma" else (hbm / HBM_PEAK_GBS), 4),
                mfma_frac=round(tf / mpeak, 4), hbm_frac=round(hbm / HBM_PEAK_GBS, 4))


def kernel_roofline(args, w, M, lib, torch, np, step, U, P, W, K, shared8=False):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")   # the HIP runtime torch already loaded
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]

    def new_event():
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    step(0)
    torch.cuda.synchronize()
    n_launch = M.moe_last_call_launches()
    names = [M.moe_launch_name(i) for i in range(n_launch)]
    evs = [(ctypes.c_void_p * (2 * n_launch))(*[new_event() for _ in range(2 * n_launch)])
           for _ in range(K)]
    try:
        for i in range(W):
            step(i)
        for i in range(K):
            M.moe_set_kernel_events(evs[i], n_launch)
            step(W + i)
        M.moe_set_kernel_events(None, 0)
        torch.cuda.synchronize()
        dur = np.zeros((K, n_launch))
        f = ctypes.c_float()
        for i in range(K):
            for j in range(n_launch):
                if hip.hipEventElapsedTime(ctypes.byref(f), evs[i][2 * j],
                                           evs[i][2 * j + 1]) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                dur[i, j] = f.value
    finally:
        M.moe_set_kernel_events(None, 0)
        for a in evs:
            for e in a:
                hip.hipEventDestroy(e)
    mean_ms = dur.mean(axis=0)
    per = ", ".join(f"{n} {m * 1e3:.2f} us" for n, m in zip(names, mean_ms))
    log(f"[bench] kernels (event-timed, mean of {K}): {per}")
    j = int(np.argmax(mean_ms))
    name, t_ms = names[j], float(mean_ms[j])
    sh = not shared8
    nv = bool(getattr(args, "nvfp4", False))
    bound, _ = kernel_work(name, w, 1, sh, nv, shared8)
    bound_kind = bound
    if bound is None:
        log(f"[bench] dominant kernel {name}: no algorithmic work model, roofline omitted")
        return None
    # per-launch work averaged over the calls the timed loop made
    if bound == "gemm":
        fl = float(np.mean([kernel_work(name, w, U[(W + i) % P], sh, nv, shared8)[1][0] for i in range(K)]))
        by = float(np.mean([kernel_work(name, w, U[(W + i) % P], sh, nv, shared8)[1][1] for i in range(K)]))
        # the bound is the resource the work needs longer at its peak
        mpeak = MFMA_PEAK_OF.get(name, MFMA_16BIT_PEAK_TFLOPS)
        bound = "mfma" if fl / (mpeak * 1e12) >= by / (HBM_PEAK_GBS * 1e9) else "hbm"
        work = fl if bound == "mfma" else by
        log(f"[bench] {name}: {fl / 1e12:.3f} TFLOP, {by / 1e9:.2f} GB unavoidable -> "
            f"bound by {bound.upper()}")
        # both fractions, whichever bounds the kernel
        both = dict(mfma_frac=round(fl / (t_ms / 1e3) / (mpeak * 1e12), 4),
                    hbm_frac=round(by / (t_ms / 1e3) / (HBM_PEAK_GBS * 1e9), 4))
    else:
        work = float(np.mean([kernel_work(name, w, U[(W + i) % P], sh, nv, shared8)[1] for i in range(K)]))
    if bound == "hbm":
        ach = work / (t_ms / 1e3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
        log(f"[bench] {name}: {t_ms * 1e3:.2f} us/launch, {work / 1e6:.2f} MB algorithmic "
            f"(mean {np.mean([U[(W + i) % P] for i in range(K)]):.2f} routed experts) -> "
            f"{ach:,.0f} GB/s")
    else:
        ach = work / (t_ms / 1e3) / 1e12
        peak, unit = MFMA_PEAK_OF.get(name, MFMA_16BIT_PEAK_TFLOPS), "TFLOP/s"
        log(f"[bench] {name}: {t_ms:.3f} ms/launch, {work / 1e12:.3f} TFLOP -> "
            f"{ach:,.1f} TFLOP/s")
    out = dict(bound=bound, achieved=round(ach, 1), peak=peak, unit=unit,
               frac=round(ach / peak, 4), traffic=recorded_traffic(name, w.name), kernel=name,
               kernel_us=round(t_ms * 1e3, 2))
    if bound_kind == "gemm":
        out.update(both)
    return out


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the counter summaries
    under profiles/ (FETCH_SIZE + WRITE_SIZE, each scaled by a copy kernel's
    reading), or None when none is recorded or the kernel's source file has
    changed since the counters were taken."""
    import glob
    import hashlib
    import re
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        text = open(path).read()
        f = dict(re.findall(r"^(kernel|workload|traffic_bytes_per_launch|kernel_source|"
                            r"kernel_source_sha256): (\S+)$", text, flags=re.M))
        if f.get("kernel") != kernel or f.get("workload") != workload:
            continue
        src = os.path.join(ROOT, f.get("kernel_source", ""))
        if not os.path.isfile(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != f.get("kernel_source_sha256"):
            log(f"[bench] {os.path.basename(path)}: kernel source changed since the counters "
                "were taken; traffic not reported")
            return None
        return int(f["traffic_bytes_per_launch"])
    return None

if __name__ == "__main__":
    sys.exit(main())
