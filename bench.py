#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

One step = one pass of the whole hot path over one batch of seeded synthetic
tokens, through the C ABI: gate GEMM + routing (moe_route), counting-sort
permutation (moe_permute), expert up and down layers (moe_expert_up,
moe_expert_down) and the weighted combine (moe_combine).  The default
workload is the Mixtral-8x7B-shaped layer (T=4096 tokens, d=4096, 8 experts,
top-2, SwiGLU 4096->14336->4096, bf16, Zipf(1.2)-skewed gate bias); every input
is resident in HBM before the timed region starts.

Prints ONE JSON line: tokens/s of the whole job (value), the roofline of the
dominant kernel (the expert up-projection grouped GEMM) from HIP events on the
stream it runs on, and the CPU oracle timed on a bounded sample of the same
workload on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                  [--no-cpu-baseline] [--mode copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec at Mixtral shape; grouped-GEMM % of bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA peaks
HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_logit_amd", "csrc", "grouped_gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(config: str):
    """HBM bytes per launch of the dominant kernel from committed counter runs,
    or None when absent or taken on a different version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(config)
    if not entry or entry.get("kernel_source_sha256_16") != source_hash(GEMM_SRC):
        return None
    return entry.get("bytes_per_launch")


def copy_mode(args):
    """Plain device copies of a known size, for scaling the HBM byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(max(args.steps, 1)):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_per_copy": n, "copies": max(args.steps, 1)}))


def cpu_baseline(case, inp, budget_s: float):
    """Oracle tokens/s on a bounded sample: gate, routing and permutation of
    all T tokens (they are needed to know the kept choices) are charged per
    token, plus the expert FFN and combine of a sample of tokens."""
    import numpy as np
    import oracle
    act = oracle.SWIGLU if case.act == "swiglu" else oracle.RELU
    t0 = time.perf_counter()
    if case.logits == "gate":
        _ze, z32 = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
    else:
        z32 = inp["logits"]
    idx, w = oracle.route(z32, case.k, case.normalize, case.lam)
    disp = oracle.dispatch(idx, case.E, oracle.capacity(case.T, case.E, case.k, case.cf))
    t_route = time.perf_counter() - t0
    threads = oracle.threads()
    g = np.random.default_rng(case.seed)
    order = g.permutation(case.T).astype(np.int32)
    n = max(threads, 1)
    t_ffn = 0.0
    done = 0
    while done < case.T:
        toks = order[done:done + n]
        t1 = time.perf_counter()
        oracle.forward_tokens(inp["x"], inp["W1"], inp["W2"], idx, w, disp["slot"], act, case.F, toks)
        t_ffn += time.perf_counter() - t1
        done += len(toks)
        if t_ffn + t_route * done / case.T >= budget_s:
            break
        n = len(toks) * 2
    per_token = t_route / case.T + t_ffn / done
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {case.T} tokens of the {case.name} layer (expert FFN + combine of the sample; "
                      f"gate, routing and permutation of all {case.T} tokens charged per token)",
            "seconds": round(t_route + t_ffn, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--mode", default="layer", choices=["layer", "copy"])
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this benchmark measures the MoE-layer forward on one GPU; multi-GPU runs are not part of it "
               "(data-parallel replicas would each run this same layer on their own tokens)")
        print(msg, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.mode == "copy":
        copy_mode(args)
        return

    import mixture_experts_layer_logit_amd as moe
    import moe_inputs

    case = moe_inputs.get(args.config)
    log(f"[bench] generating inputs for {case.name}")
    inp = moe_inputs.make(case)
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    dt = torch.float32 if case.dtype == "f32" else torch.bfloat16

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    T, d, E, k, F = case.T, case.d, case.E, case.k, case.F
    n1 = 2 * F if case.act == "swiglu" else F
    p = moe.problem(T, d, E, k, F, act=case.act, dtype=case.dtype, normalize=case.normalize, lam=case.lam,
                    cf=case.cf)
    with torch.cuda.stream(stream):
        x = dev(inp["x"])
        Wg = dev(inp["Wg"]) if inp["Wg"] is not None else None
        bg = dev(inp["bg"]) if inp["bg"] is not None else None
        W1 = dev(inp["W1"])
        W2 = dev(inp["W2"])
        logits = dev(inp["logits"]) if case.logits == "given" else torch.empty(T, E, dtype=torch.float32,
                                                                               device="cuda")
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, dtype=torch.float32, device="cuda")
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        slot = torch.empty(T, k, dtype=torch.int32, device="cuda")
        src = torch.empty(T * k, dtype=torch.int32, device="cuda")
        h = torch.empty(T * k, F, dtype=dt, device="cuda")
        y_perm = torch.empty(T * k, d, dtype=dt, device="cuda")
        y = torch.empty(T, d, dtype=dt, device="cuda")
        ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    s = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        moe.moe_route(p, x if Wg is not None else None, Wg, bg, logits, idx, w, stream=s)
        if ev is not None:
            ev[1].record(stream)
        # no x_perm copy: the up projection gathers the rows of x through src
        moe.moe_permute(p, idx, None, counts, offsets, slot, src, None, ws, stream=s)
        if ev is not None:
            ev[2].record(stream)
        moe.moe_expert_up(p, x, src, offsets, W1, h, ws=ws, stream=s)
        if ev is not None:
            ev[3].record(stream)
        moe.moe_expert_down(p, h, offsets, W2, y_perm, ws=ws, stream=s)
        if ev is not None:
            ev[4].record(stream)
        moe.moe_combine(p, y_perm, slot, w, y, stream=s)
        if ev is not None:
            ev[5].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    names = ["route", "permute", "expert_up", "expert_down", "combine"]
    stage_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events])) for i, n in enumerate(names)}
    P = int(offsets[-1].item())
    dropped = T * k - P
    up_flops = 2.0 * P * d * n1
    down_flops = 2.0 * P * F * d
    gate_flops = 2.0 * T * d * E if case.logits == "gate" else 0.0
    ms_per_step = elapsed * 1e3 / args.steps
    peak = PEAK_TFLOPS[case.dtype]
    up_tflops = up_flops / (stage_ms["expert_up"] * 1e-3) / 1e12
    ffn_tflops = (up_flops + down_flops) / ((stage_ms["expert_up"] + stage_ms["expert_down"]) * 1e-3) / 1e12
    row_bytes = d * (4 if case.dtype == "f32" else 2)
    combine_gbps = (T + P) * row_bytes / (stage_ms["combine"] * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": f"{case.name}: T={T} d={d} E={E} k={k} F={F} {case.act} {case.dtype}"
                               + (f" lambda-normalised" if case.normalize else "")
                               + (f" cf={case.cf}" if case.cf > 0 else " dropless")
                               + (" Zipf(1.2) gate bias" if case.bias == "zipf" else ""),
                   "T": T, "d": d, "E": E, "k": k, "F": F, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": up_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": up_tflops / peak, "traffic": stored_traffic(case.name),
                     "kernel": "moe_grouped_gemm_kernel (expert up-projection + activation)"},
        "tflops": (up_flops + down_flops + gate_flops) / (ms_per_step * 1e-3) / 1e12,
        "grouped_gemm_pct_of_bf16_peak": 100.0 * ffn_tflops / peak,
        "stage_ms": stage_ms,
        "combine_hbm_frac": combine_gbps / HBM_GBPS,
        "kept_rows": P,
        "dropped_assignments": dropped,
        "expert_loads": counts.cpu().tolist(),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(case, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
