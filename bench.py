#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

One step = one moe_forward call (the whole hot path: gate GEMM, routing,
counting-sort permutation, expert up and down layers, weighted combine) over
one batch of seeded synthetic tokens, through the C ABI, with every input
resident in HBM before the timed region starts.  The default workload is the
Mixtral-8x7B-shaped layer (T=4096 tokens, d=4096, 8 experts, top-2, SwiGLU
4096->14336->4096, bf16, Zipf(1.2)-skewed gate bias).

`value` is T divided by the median of the per-step HIP-event times of
moe_forward (W warm-up calls, then K timed calls, K >= 50 by default); the
timed calls are also bracketed by device synchronisations and their wall
clock reported.  A separate pass times the five entry points one by one
(moe_route, moe_permute, moe_expert_up, moe_expert_down, moe_combine) for the
per-stage breakdown and the roofline of the dominant kernel (the expert
up-projection grouped GEMM with its split-K reduction).  The CPU oracle is
timed on this host's cores: a bounded sample of the Mixtral layer for the
headline line, and per workload below.

Also on the line: the same expert GEMMs through the vendor library (one
hipBLASLt product per expert, for reference), a device-to-device copy's bandwidth (the HBM reference),
the standalone permutation with its row copy (moe_permute writing x_perm)
and the combine alone (both per launch, from batches of launches between
two events, so the events' own cost is spread), the router statistics, a shared expert, the layer with FP8 expert weights and
the training step ("next_rows"), and every other workload ("other_configs":
moe_forward median, stage breakdown, roofline against the bound that applies,
and a CPU-oracle baseline; routing inputs from the seeded generator, expert
weights drawn on the device with the same distribution, since their values
do not change the work).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                  [--no-cpu-baseline] [--no-other-configs] [--no-next-rows]
                  [--mode copy|train]

--mode train times only the training step and prints its own JSON line (for
profiling the backward); --mode copy runs plain device copies (the HBM
counter calibration).
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
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}   # MI355X dense MFMA peaks
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
    flops = case.ffn_flops_dropless * (disp["P"] / (case.T * case.k)) + (
        2.0 * case.T * case.d * case.E if case.logits == "gate" else 0.0)
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "gflops": flops / case.T / per_token / 1e9,
            "sample": f"{done} of {case.T} tokens of the {case.name} layer (expert FFN + combine of the sample; "
                      f"gate, routing and permutation of all {case.T} tokens charged per token)",
            "seconds": round(t_route + t_ffn, 2)}


def cpu_baseline_full(case, inp, reps: int = 3):
    """Oracle tokens/s of whole forwards (gate, routing, permutation, expert
    FFN and combine of every token), best of `reps`."""
    import oracle
    act = oracle.SWIGLU if case.act == "swiglu" else oracle.RELU
    best = None
    for _ in range(reps):
        t0 = time.perf_counter()
        if case.logits == "gate":
            _ze, z32 = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
        else:
            z32 = inp["logits"]
        idx, w = oracle.route(z32, case.k, case.normalize, case.lam)
        disp = oracle.dispatch(idx, case.E, oracle.capacity(case.T, case.E, case.k, case.cf))
        oracle.forward_tokens(inp["x"], inp["W1"], inp["W2"], idx, w, disp["slot"], act, case.F)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    flops = case.ffn_flops_dropless * (disp["P"] / (case.T * case.k)) + (
        2.0 * case.T * case.d * case.E if case.logits == "gate" else 0.0)
    return {"value": case.T / best, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "gflops": flops / best / 1e9,
            "sample": f"whole forward of all {case.T} tokens of the {case.name} layer, best of {reps}",
            "seconds": round(best, 3)}


def copy_bandwidth(stream, n=1 << 30, reps=10):
    """Achieved bandwidth of a plain device-to-device copy of n bytes (read n,
    write n), HIP events on the stream; the reference for the HBM fractions."""
    import numpy as np
    import torch
    with torch.cuda.stream(stream):
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            b.copy_(a)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            b.copy_(a)
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
    del a, b
    return {"gbps": 2.0 * n / (ms * 1e-3) / 1e9, "bytes_moved": 2 * n, "ms": ms,
            "frac_of_8TBps": 2.0 * n / (ms * 1e-3) / 1e9 / HBM_GBPS}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--mode", default="layer", choices=["layer", "copy", "train"])
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

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    case = moe_inputs.get(args.config)
    log(f"[bench] generating inputs for {case.name}")
    inp = moe_inputs.make(case)
    with torch.cuda.stream(stream):
        dev_w = {"W1": to_dev(inp["W1"]), "W2": to_dev(inp["W2"])}
    lay = Layer(moe, case, inp, dev_w, stream)
    if args.mode == "train":  # the training step alone (forward keeping intermediates, backward)
        log("[bench] training step")
        r = lay.time_train(args.steps)
        r.update(workload=workload_name(case), steps=args.steps)
        print(json.dumps(r), flush=True)
        return
    log(f"[bench] moe_forward: {args.warmup} warm-up + {args.steps} timed steps")
    fwd = lay.time_forward(args.steps, args.warmup)
    log("[bench] stage pass")
    res = lay.time(args.steps, args.warmup)
    T, d, E, k, F = case.T, case.d, case.E, case.k, case.F
    stage_ms, P = res["stage_ms"], res["P"]
    ms_per_step = fwd["median_ms"]
    peak = PEAK_TFLOPS[case.dtype]
    up_tflops = lay.up_flops(P) / (stage_ms["expert_up"] * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
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
        "config": {"workload": workload_name(case), "T": T, "d": d, "E": E, "k": k, "F": F,
                   "parallelism": "single GPU"},
        "timing": {"entry_point": "moe_forward", "stat": f"median of {args.steps} HIP-event step times after "
                   f"{args.warmup} warm-ups", "mean_ms": fwd["mean_ms"], "min_ms": fwd["min_ms"],
                   "wall_ms_per_step": fwd["wall_ms"],
                   "stage_sum_ms": sum(stage_ms.values()),
                   "stage_sum_vs_forward": sum(stage_ms.values()) / ms_per_step},
        "roofline": {"bound": "mfma", "achieved": up_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": up_tflops / peak, "traffic": stored_traffic(case.name),
                     "kernel": "moe_expert_up: moe_grouped_gemm_kernel (up-projection + activation) and its K-split reduction"},
    }
    result.update(lay.summary(res, ms_per_step))
    log("[bench] copy bandwidth, standalone permutation with its row copy")
    result["copy_bandwidth"] = copy_bandwidth(stream)
    result["permute_row_copy"] = lay.time_permute_copy(args.steps)
    result["combine_alone"] = lay.time_combine_alone()
    if case.dtype == "bf16":
        log("[bench] the expert GEMMs through the vendor library, for reference")
        ref = lay.time_library_reference()
        ref["ours_vs_library_up"] = ref["up"]["ms"] / stage_ms["expert_up"]
        ref["ours_vs_library_down"] = ref["down"]["ms"] / stage_ms["expert_down"]
        result["library_reference"] = ref
    if not args.no_graph:
        result["graph_replay"] = lay.time_graph(args.steps)

    # rows beyond the layer step: router statistics, shared expert
    if not args.no_next_rows:
        log("[bench] router statistics and shared expert")
        result["next_rows"] = lay.time_next_rows(min(args.steps, 20), res)

    if not args.no_other_configs:
        others = {}
        for name in moe_inputs.FULL:
            if name == case.name:
                continue
            c = moe_inputs.get(name)
            log(f"[bench] {name}: routing inputs from the seeded generator, expert weights drawn on the device")
            ri = moe_inputs.make(c, weights=False)
            gen = torch.Generator(device="cuda")
            gen.manual_seed(c.seed)
            n1 = 2 * c.F if c.act == "swiglu" else c.F
            dt = torch.float32 if c.dtype == "f32" else torch.bfloat16
            with torch.cuda.stream(stream):
                w = {"W1": (torch.randn(c.E, n1, c.d, generator=gen, device="cuda") * c.w_std).to(dt),
                     "W2": (torch.randn(c.E, c.d, c.F, generator=gen, device="cuda") * c.w_std).to(dt)}
            lo = Layer(moe, c, ri, w, stream)
            f = lo.time_forward(args.steps, args.warmup)
            r = lo.time(max(args.steps // 2, 10), 2)
            msps = f["median_ms"]
            o = {"workload": workload_name(c), "tokens_per_s": c.T / (msps * 1e-3), "ms_per_step": msps,
                 "mean_ms": f["mean_ms"], "stage_sum_ms": sum(r["stage_ms"].values())}
            o.update(lo.summary(r, msps))
            o["roofline"] = lo.roofline(r)
            if not args.no_graph:
                o["graph_replay"] = lo.time_graph(max(args.steps // 2, 10))
            if not args.no_cpu_baseline:
                # the oracle's arithmetic does not depend on the weights'
                # values: it runs on host copies of the device weights
                torch.cuda.synchronize()
                ri["W1"], ri["W2"] = to_host(w["W1"]), to_host(w["W2"])
                log(f"[bench] {name}: timing the CPU oracle")
                if name in ("skywork_m", "skywork_m_zipf"):
                    o["cpu_baseline"] = cpu_baseline(c, ri, args.cpu_seconds / 2)
                else:
                    o["cpu_baseline"] = cpu_baseline_full(c, ri, 3)
            others[name] = o
            del lo, w, ri
            torch.cuda.empty_cache()
        result["other_configs"] = others

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(case, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def to_host(t):
    import numpy as np
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def to_dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def workload_name(case):
    return (f"{case.name}: T={case.T} d={case.d} E={case.E} k={case.k} F={case.F} {case.act} {case.dtype}"
            + (" lambda-normalised" if case.normalize else "")
            + (f" cf={case.cf}" if case.cf > 0 else " dropless")
            + (" Zipf(1.2) gate bias" if case.bias == "zipf" else "")
            + (" given logits" if case.logits == "given" else ""))


class Layer:
    """Device buffers and the timed step of one workload.  One step = one
    moe_forward call: gate + routing, permutation (indices only: the up
    projection gathers the token rows itself), expert up and down layers,
    weighted combine, all on one stream.  The stage pass calls the five entry
    points of the same step one by one with an event between them."""

    NAMES = ["route", "permute", "expert_up", "expert_down", "combine"]

    def __init__(self, moe, case, inp, w, stream):
        import torch
        self.moe, self.case, self.stream = moe, case, stream
        T, d, E, k, F = case.T, case.d, case.E, case.k, case.F
        self.n1 = 2 * F if case.act == "swiglu" else F
        self.p = moe.problem(T, d, E, k, F, act=case.act, dtype=case.dtype, normalize=case.normalize,
                             lam=case.lam, cf=case.cf)
        dt = torch.float32 if case.dtype == "f32" else torch.bfloat16
        self.dt = dt
        with torch.cuda.stream(stream):
            self.x = to_dev(inp["x"])
            self.Wg = to_dev(inp["Wg"]) if inp.get("Wg") is not None else None
            self.bg = to_dev(inp["bg"]) if inp.get("bg") is not None else None
            self.W1, self.W2 = w["W1"], w["W2"]
            self.logits = to_dev(inp["logits"]) if case.logits == "given" else \
                torch.empty(T, E, dtype=torch.float32, device="cuda")
            self.idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
            self.w = torch.empty(T, k, dtype=torch.float32, device="cuda")
            self.counts = torch.empty(E, dtype=torch.int32, device="cuda")
            self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
            self.slot = torch.empty(T, k, dtype=torch.int32, device="cuda")
            self.src = torch.empty(T * k, dtype=torch.int32, device="cuda")
            self.h = torch.empty(T * k, F, dtype=dt, device="cuda")
            self.y_perm = torch.empty(T * k, d, dtype=dt, device="cuda")
            self.y = torch.empty(T, d, dtype=dt, device="cuda")
            self.ws = torch.empty(moe.moe_workspace_size(self.p), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def step(self, ev=None):
        moe, p, s = self.moe, self.p, self.stream.cuda_stream
        rec = (lambda i: ev[i].record(self.stream)) if ev is not None else (lambda i: None)
        rec(0)
        moe.moe_route(p, self.x if self.Wg is not None else None, self.Wg, self.bg, self.logits, self.idx, self.w,
                      stream=s)
        rec(1)
        moe.moe_permute(p, self.idx, None, self.counts, self.offsets, self.slot, self.src, None, self.ws, stream=s)
        rec(2)
        moe.moe_expert_up(p, self.x, self.src, self.offsets, self.W1, self.h, ws=self.ws, stream=s)
        rec(3)
        moe.moe_expert_down(p, self.h, self.offsets, self.W2, self.y_perm, ws=self.ws, stream=s)
        rec(4)
        moe.moe_combine(p, self.y_perm, self.slot, self.w, self.y, stream=s)
        rec(5)

    def forward(self):
        """One moe_forward call (the step), with the routing outputs kept in
        the step's buffers."""
        moe, p, s = self.moe, self.p, self.stream.cuda_stream
        info = {"topk_idx": self.idx, "topk_w": self.w, "counts": self.counts, "offsets": self.offsets,
                "slot": self.slot, "src_token": self.src}
        moe.moe_forward(p, self.x, self.Wg, self.bg, self.W1, self.W2, self.y, logits=self.logits, info=info,
                        ws=self.ws, stream=s)

    def time_forward(self, steps, warmup):
        """moe_forward: warm-ups, then `steps` calls with a HIP event after
        each on the layer's stream, the whole timed region bracketed by device
        synchronisations."""
        import numpy as np
        import torch
        for _ in range(warmup):
            self.forward()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(self.stream)
        for i in range(steps):
            self.forward()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
        return {"median_ms": float(np.median(ms)), "mean_ms": float(ms.mean()), "min_ms": float(ms.min()),
                "wall_ms": wall * 1e3 / steps}

    def time_batched(self, call, reps=5, batch=10):
        """Per-launch time of a short call: events around `batch` calls in a
        row (so the events' own cost is spread over them), median of `reps`."""
        import numpy as np
        import torch
        for _ in range(3):
            call()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(self.stream)
        for i in range(reps):
            for _ in range(batch):
                call()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])) / batch

    def time_combine_alone(self):
        """moe_combine on the step's y_perm and routing, launched back to back.
        Algorithmic bytes: the kept rows of y_perm read, y written, 8 T k of
        slot and weight."""
        c, s = self.case, self.stream.cuda_stream
        ms = self.time_batched(lambda: self.moe.moe_combine(self.p, self.y_perm, self.slot, self.w, self.y,
                                                            stream=s))
        P = int(self.offsets[-1].item())
        b = 4 if c.dtype == "f32" else 2
        byts = (c.T + P) * c.d * b + 8.0 * c.T * c.k
        return {"us": ms * 1e3, "bytes": byts, "gbps": byts / (ms * 1e-3) / 1e9,
                "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_GBPS,
                "note": "per launch, 10 launches between two HIP events, median of 5"}

    def time_permute_copy(self, steps):
        """moe_permute with its row copy (x_perm written, the path moe_forward
        takes when x is beyond the fused gather's 32-bit offsets), on the
        step's routing.  Algorithmic bytes: x read once, P rows written, plus
        the index traffic (12 T k)."""
        import numpy as np
        import torch
        moe, p, c, s = self.moe, self.p, self.case, self.stream.cuda_stream
        with torch.cuda.stream(self.stream):
            xp = torch.empty(c.T * c.k, c.d, dtype=self.dt, device="cuda")
        call = lambda: moe.moe_permute(p, self.idx, self.x, self.counts, self.offsets, self.slot, self.src, xp,  # noqa
                                       self.ws, stream=s)
        ms = self.time_batched(call, reps=max(steps // 10, 5))
        P = int(self.offsets[-1].item())
        b = 4 if c.dtype == "f32" else 2
        byts = (c.T + P) * c.d * b + 12.0 * c.T * c.k
        del xp
        return {"ms": ms, "bytes": byts, "gbps": byts / (ms * 1e-3) / 1e9,
                "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_GBPS,
                "note": "count + scan + scatter + row gather kernels of one moe_permute call with x_perm; "
                        "per call, 10 calls between two HIP events, median"}

    def roofline(self, res):
        """Roofline of the grouped GEMM (up + down) and of the step:
        frac = max(t_flops, t_bytes) / t, with t_flops at the dtype's MFMA peak
        and t_bytes the algorithmic HBM bytes (expert weights, the activation
        rows read, h written and read back, y_perm written) at 8 TB/s; bound
        names the larger of the two."""
        c = self.case
        stage_ms, P = res["stage_ms"], res["P"]
        b = 4 if c.dtype == "f32" else 2
        flops = self.up_flops(P) + 2.0 * P * c.F * c.d
        wbytes = c.E * (self.n1 * c.d + c.d * c.F) * b
        byts = wbytes + P * c.d * b + 2.0 * P * c.F * b + P * c.d * b
        t = (stage_ms["expert_up"] + stage_ms["expert_down"]) * 1e-3
        t_f = flops / (PEAK_TFLOPS[c.dtype] * 1e12)
        t_b = byts / (HBM_GBPS * 1e9)
        return {"kernel": "grouped GEMM, up + down (with their K-split reductions)",
                "bound": "mfma" if t_f >= t_b else "hbm", "frac": max(t_f, t_b) / t,
                "t_flops_us": t_f * 1e6, "t_bytes_us": t_b * 1e6, "measured_us": t * 1e6,
                "flops": flops, "bytes": byts, "mfma_frac": t_f / t, "hbm_frac": t_b / t}

    def time(self, steps, warmup):
        """The stage pass: the five entry points of the step called one by
        one with an event between them; per-stage medians."""
        import numpy as np
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(events[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        stage_ms = {n: float(np.median([e[i].elapsed_time(e[i + 1]) for e in events]))
                    for i, n in enumerate(self.NAMES)}
        return {"stage_ms": stage_ms, "elapsed": elapsed, "P": int(self.offsets[-1].item())}

    def time_graph(self, steps):
        """The same step (moe_forward) captured once in a HIP graph (every
        entry point only launches kernels on the given stream) and replayed:
        the step without the host's per-launch cost."""
        import numpy as np
        import torch
        self.forward()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            self.forward()
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        with torch.cuda.stream(self.stream):
            ev[0].record(self.stream)
            for i in range(steps):
                g.replay()
                ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
        del g
        return {"ms_per_step": ms, "tokens_per_s": self.case.T / (ms * 1e-3)}

    def up_flops(self, P):
        return 2.0 * P * self.case.d * self.n1

    def summary(self, res, ms_per_step):
        c = self.case
        stage_ms, P = res["stage_ms"], res["P"]
        up, down = self.up_flops(P), 2.0 * P * c.F * c.d
        gate = 2.0 * c.T * c.d * c.E if c.logits == "gate" else 0.0
        peak = PEAK_TFLOPS[c.dtype]
        ffn_ms = stage_ms["expert_up"] + stage_ms["expert_down"]
        b = 4 if c.dtype == "f32" else 2
        combine_bytes = (c.T + P) * c.d * b + 8.0 * c.T * c.k
        return {
            "tflops": (up + down + gate) / (ms_per_step * 1e-3) / 1e12,
            "grouped_gemm_pct_of_peak": 100.0 * (up + down) / (ffn_ms * 1e-3) / 1e12 / peak,
            "stage_ms": stage_ms,
            "combine_hbm_frac": combine_bytes / (stage_ms["combine"] * 1e-3) / 1e9 / HBM_GBPS,
            "kept_rows": P,
            "dropped_assignments": c.T * c.k - P,
            "expert_loads": self.counts.cpu().tolist() if c.E <= 64 else
            {"min": int(self.counts.min()), "max": int(self.counts.max())},
        }

    def time_library_reference(self, reps=10):
        """The same expert GEMMs through the vendor library, for reference:
        one torch F.linear (hipBLASLt, bf16 in, fp32 accumulate) per expert
        over that expert's permuted rows, no activation, with the step's
        routing; the up-projection's 8 products then the down-projection's,
        HIP events around each sequence on the layer's stream.  It reads a
        permuted copy of x (made before the timed region) where the library
        path cannot gather, and it writes u and the outputs without the
        activation, so it does slightly less work than moe_expert_up."""
        import numpy as np
        import torch
        import torch.nn.functional as Fn
        c = self.case
        off = [int(v) for v in self.offsets.cpu()]
        with torch.cuda.stream(self.stream):
            xp = self.x.index_select(0, self.src[:off[-1]].long())
            u = torch.empty(off[-1], self.n1, dtype=self.dt, device="cuda")
            hh = torch.empty(off[-1], c.F, dtype=self.dt, device="cuda")
            yp = torch.empty(off[-1], c.d, dtype=self.dt, device="cuda")

        def up():
            for e in range(c.E):
                if off[e + 1] > off[e]:
                    torch.matmul(xp[off[e]:off[e + 1]], self.W1[e].t(), out=u[off[e]:off[e + 1]])

        def down():
            for e in range(c.E):
                if off[e + 1] > off[e]:
                    torch.matmul(hh[off[e]:off[e + 1]], self.W2[e].t(), out=yp[off[e]:off[e + 1]])
        out = {}
        P = off[-1]
        for name, fn, flops in (("up", up, 2.0 * P * c.d * self.n1), ("down", down, 2.0 * P * c.F * c.d)):
            with torch.cuda.stream(self.stream):
                for _ in range(3):
                    fn()
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
                ev[0].record(self.stream)
                for i in range(reps):
                    fn()
                    ev[i + 1].record(self.stream)
            torch.cuda.synchronize()
            ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
            out[name] = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
                         "frac_of_peak": flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[c.dtype]}
        del xp, u, hh, yp
        out["note"] = ("hipBLASLt through torch.matmul, one product per expert over its permuted rows "
                       "(A contiguous, W[e] read as stored, no activation); median of %d sequences" % reps)
        return out

    def time_next_rows(self, steps, res):
        """Router statistics on the step's routing; a shared expert of width F
        over all tokens and the combine that adds it."""
        import numpy as np
        import torch
        moe, p, c, s = self.moe, self.p, self.case, self.stream.cuda_stream
        T, d, E, F = c.T, c.d, c.E, c.F
        b = 4 if c.dtype == "f32" else 2
        with torch.cuda.stream(self.stream):
            frac = torch.empty(E, dtype=torch.float32, device="cuda")
            mp = torch.empty(E, dtype=torch.float32, device="cuda")
            sc = torch.empty(3, dtype=torch.float32, device="cuda")
            Fs = F
            n1s = 2 * Fs if c.act == "swiglu" else Fs
            gen = torch.Generator(device="cuda")
            gen.manual_seed(c.seed + 7)
            Ws1 = (torch.randn(n1s, d, generator=gen, device="cuda") * c.w_std).to(self.dt)
            Ws2 = (torch.randn(d, Fs, generator=gen, device="cuda") * c.w_std).to(self.dt)
            ysh = torch.empty(T, d, dtype=self.dt, device="cuda")
            sws = torch.empty(moe.moe_shared_workspace_size(p, Fs), dtype=torch.uint8, device="cuda")
        calls = {
            "router_stats": lambda: moe.moe_router_stats(p, self.logits, self.counts, self.offsets, frac, mp, sc,
                                                         self.ws, stream=s),
            "shared_expert": lambda: moe.moe_shared_expert(p, Fs, self.x, Ws1, Ws2, ysh, sws, stream=s),
            "combine_shared": lambda: moe.moe_combine_shared(p, self.y_perm, self.slot, self.w, ysh, self.y,
                                                             stream=s),
        }
        out = {}
        for name, fn in calls.items():
            for _ in range(2):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            ev[0].record(self.stream)
            for i in range(steps):
                fn()
                ev[i + 1].record(self.stream)
            torch.cuda.synchronize()
            out[name] = {"ms": float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))}
        P = res["P"]
        st = out["router_stats"]
        st["bytes"] = 4.0 * T * E + 8.0 * E + 12
        st["hbm_frac"] = st["bytes"] / (st["ms"] * 1e-3) / 1e9 / HBM_GBPS
        st["values"] = {"aux": float(sc[0]), "z_loss": float(sc[1]), "drop_rate": float(sc[2])}
        sh = out["shared_expert"]
        sh["Fs"] = Fs
        sh["tflops"] = (2.0 * T * d * n1s + 2.0 * T * Fs * d) / (sh["ms"] * 1e-3) / 1e12
        sh["mfma_frac"] = sh["tflops"] / PEAK_TFLOPS[c.dtype]
        cs = out["combine_shared"]
        cs["bytes"] = (P + 2 * T) * d * b + 8.0 * T * c.k
        cs["hbm_frac"] = cs["bytes"] / (cs["ms"] * 1e-3) / 1e9 / HBM_GBPS
        del Ws1, Ws2, ysh, sws
        if c.dtype == "bf16" and d % 128 == 0 and F % 128 == 0:
            out["fp8_layer"] = self.time_fp8(steps)
        out["backward"] = self.time_train(steps)
        return out

    def time_train(self, steps):
        """Training step: moe_forward_train (the forward keeping u, h and
        y_perm), then moe_backward on a seeded incoming gradient dy; each call
        timed with events on the layer's stream."""
        import numpy as np
        import torch
        import moe_inputs
        moe, p, c, s = self.moe, self.p, self.case, self.stream.cuda_stream
        T, d, E, k, F = c.T, c.d, c.E, c.k, c.F
        n1, dt = self.n1, self.dt
        with torch.cuda.stream(self.stream):
            dy = to_dev(moe_inputs.make_dy(c))
            saved = {"u": torch.empty(T * k, n1, dtype=dt, device="cuda"), "h": self.h, "y_perm": self.y_perm}
            info = {"topk_idx": self.idx, "topk_w": self.w, "counts": self.counts, "offsets": self.offsets,
                    "slot": self.slot, "src_token": self.src}
            bws = torch.empty(moe.moe_backward_workspace_size(p), dtype=torch.uint8, device="cuda")
            dx = torch.empty(T, d, dtype=dt, device="cuda")
            dW1 = torch.empty(E, n1, d, dtype=torch.float32, device="cuda")
            dW2 = torch.empty(E, d, F, dtype=torch.float32, device="cuda")
            gate = self.Wg is not None
            dWg = torch.empty(E, d, dtype=torch.float32, device="cuda") if gate else None
            dbg = torch.empty(E, dtype=torch.float32, device="cuda") if gate else None
        torch.cuda.synchronize()

        def fwd():
            moe.moe_forward_train(p, self.x, self.Wg, self.bg, self.W1, self.W2, self.y, self.logits, info, saved,
                                  self.ws, stream=s)

        def bwd():
            moe.moe_backward(p, dy, self.x, self.Wg, self.W1, self.W2, self.logits, info, saved, dx, dWg, dbg, dW1,
                             dW2, bws, stream=s)

        for _ in range(2):
            fwd()
            bwd()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(self.stream)
            fwd()
            ev[i][1].record(self.stream)
            bwd()
            ev[i][2].record(self.stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        P = int(self.offsets[-1].item())
        # algorithmic FLOPs: input and weight gradients of both expert layers
        # over the kept rows (the zero padding of the weight-gradient GEMMs' K
        # is not counted), and the gate's two [T,E]x[E,d]-sized products
        bwd_gemm = 2.0 * (2.0 * P * d * (n1 + F))
        gate_f = 4.0 * T * E * d if gate else 0.0
        peak = PEAK_TFLOPS[c.dtype]
        return {
            "tokens_per_s": T * steps / elapsed,
            "ms_per_step": elapsed * 1e3 / steps,
            "forward_train_ms": f_ms,
            "backward_ms": b_ms,
            "backward_tflops": (bwd_gemm + gate_f) / (b_ms * 1e-3) / 1e12,
            "backward_frac_of_peak": (bwd_gemm + gate_f) / (b_ms * 1e-3) / 1e12 / peak,
            "flops_note": "backward: 2 x the forward expert FLOPs (input and weight gradients) + 4 T E d for the gate",
        }

    def time_fp8(self, steps):
        """The same layer with FP8 (E4M3) expert weights and activations: the
        bf16 weights are quantised on the device, then the FP8 step (route,
        permute, quantise x, FP8 up, quantise h, FP8 down, combine) is timed
        stage by stage."""
        import numpy as np
        import torch
        moe, p, c, s = self.moe, self.p, self.case, self.stream.cuda_stream
        T, d, E, k, F = c.T, c.d, c.E, c.k, c.F
        n1 = self.n1
        with torch.cuda.stream(self.stream):
            W1q = torch.empty(E, n1, d, dtype=torch.uint8, device="cuda")
            w1s = torch.empty(E, n1, dtype=torch.float32, device="cuda")
            W2q = torch.empty(E, d, F, dtype=torch.uint8, device="cuda")
            w2s = torch.empty(E, d, dtype=torch.float32, device="cuda")
            moe.moe_quantize_fp8(self.W1.view(E * n1, d), W1q.view(E * n1, d), w1s.view(-1), stream=s)
            moe.moe_quantize_fp8(self.W2.view(E * d, F), W2q.view(E * d, F), w2s.view(-1), stream=s)
            xq = torch.empty(T, d, dtype=torch.uint8, device="cuda")
            xs = torch.empty(T, dtype=torch.float32, device="cuda")
            hq = torch.empty(T * k, F, dtype=torch.uint8, device="cuda")
            hs = torch.empty(T * k, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        names = ["route", "permute", "quantize_x", "expert_up", "quantize_h", "expert_down", "combine"]

        def step(ev=None):
            rec = (lambda i: ev[i].record(self.stream)) if ev is not None else (lambda i: None)
            rec(0)
            moe.moe_route(p, self.x if self.Wg is not None else None, self.Wg, self.bg, self.logits, self.idx,
                          self.w, stream=s)
            rec(1)
            moe.moe_permute(p, self.idx, None, self.counts, self.offsets, self.slot, self.src, None, self.ws,
                            stream=s)
            rec(2)
            moe.moe_quantize_fp8(self.x, xq, xs, stream=s)
            rec(3)
            moe.moe_expert_up_fp8(p, xq, xs, self.src, self.offsets, W1q, w1s, self.h, ws=self.ws, stream=s)
            rec(4)
            moe.moe_quantize_fp8(self.h, hq, hs, stream=s)
            rec(5)
            moe.moe_expert_down_fp8(p, hq, hs, self.offsets, W2q, w2s, self.y_perm, ws=self.ws, stream=s)
            rec(6)
            moe.moe_combine(p, self.y_perm, self.slot, self.w, self.y, stream=s)
            rec(7)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            step(events[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        stage_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events])) for i, n in enumerate(names)}
        P = int(self.offsets[-1].item())
        up, down = 2.0 * P * d * n1, 2.0 * P * F * d
        peak = PEAK_TFLOPS["fp8"]
        return {
            "tokens_per_s": T * steps / elapsed,
            "ms_per_step": elapsed * 1e3 / steps,
            "stage_ms": stage_ms,
            "up_tflops": up / (stage_ms["expert_up"] * 1e-3) / 1e12,
            "up_frac_of_fp8_peak": up / (stage_ms["expert_up"] * 1e-3) / 1e12 / peak,
            "grouped_gemm_pct_of_fp8_peak": 100.0 * (up + down) / ((stage_ms["expert_up"] + stage_ms["expert_down"])
                                                                   * 1e-3) / 1e12 / peak,
            "weights": "E4M3 codes with power-of-two row scales, quantised on the device from the bf16 weights",
        }


if __name__ == "__main__":
    main()
