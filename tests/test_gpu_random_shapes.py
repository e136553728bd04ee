"""GPU parity on seeded random layer shapes, beyond the named workloads.

Each case draws T, d, E, k, F, the activation, the dtype, the normalisation,
λ, the capacity factor and the logits source from its own seed (d and F
multiples of 64, k <= min(E, 8)), so the tile configurations, partial tiles,
capacity drops, empty experts and the K-split tail all meet shapes no named
workload has.  Per case:
  * the forward (moe_forward) and the training forward (moe_forward_train)
    give bit-identical routing and outputs;
  * gate logits lie within the rigorous bound of the exact fp64 logits
    (tests/_margins.py);
  * routing, counts, offsets, slots and source tokens equal the oracle's on
    the GPU's fp32 logits, bit for bit (the plainest-reading contract: the
    oracle takes the GPU's logits for parity, so near-ties of random gate
    weights need no exclusion);
  * y, dx, dW1, dW2, dWg and dbg meet the max-abs-rel bar against the oracle
    (ReLU decisions within the fp32 accumulation bound get the allowance of
    the backward tests).
The gate gradients are sums over tokens of per-token logit gradients dz[t,e]
(dbg_e = sum_t dz[t,e], dWg[e,i] = sum_t dz[t,e] x[t,i]); each dz[t] carries
the error that the layer's bf16 storage of h and y_perm puts into <dy, o>
(about 2^-8 relative, two roundings).  When the terms cancel (few experts
under the normalisation, whose 1/sigma amplifies single tokens) the sum's
error follows the terms, not the sum, so those two outputs also get an
allowance of 2^-7 sum_t |dz[t,e]| (|x[t,i]|): twice the storage rounding,
still far below what a wrong term in the formula would move (the scale of
the terms themselves).  An emulation of the bf16 storage in fp64 reproduced
the GPU's dbg to 1e-5 on the case that needed it.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_logit_amd as moe
import moe_inputs
import oracle
from _gpu import TOL, TOPK_W_ATOL, dev, host, maxrel, problem_of, run_train, to_f64, torch_dtype, within
from _margins import logit_eps, relu_unpinned
from _fp8_bound import fp8_code_allowance

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

N_CASES = 24


def random_case(i):
    g = np.random.default_rng([7717, i])
    E = int(g.choice([1, 2, 3, 5, 8, 13, 16, 33, 64]))
    k = int(g.integers(1, min(E, 8) + 1))
    return moe_inputs.Case(
        name=f"rand{i}",
        T=int(g.choice([1, 2, 7, 64, 129, 300, 777])),
        d=64 * int(g.integers(1, 9)),
        E=E, k=k,
        F=64 * int(g.integers(1, 9)),
        act=str(g.choice(["relu", "swiglu"])),
        dtype=str(g.choice(["bf16", "bf16", "f32"])),
        seed=7717 * 1000 + i,
        normalize=bool(g.integers(0, 2)),
        lam=float(g.choice([0.5, 1.0, 2.0])),
        cf=float(g.choice([0.0, 0.0, 0.5, 1.0, 1.25, 3.0])),
        logits=str(g.choice(["gate", "gate", "given"])),
        x_std=1.0, w_std=0.05, wg_std=0.05)


def act_code(case):
    return oracle.SWIGLU if case.act == "swiglu" else oracle.RELU


def forward_only(case, inp):
    """moe_forward's routing and output (host copies)."""
    p = problem_of(case)
    T, E, k, d = case.T, case.E, case.k, case.d
    gate = inp.get("Wg") is not None
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda") if gate else dev(inp["logits"])
    info = {"topk_idx": torch.empty(T, k, dtype=torch.int32, device="cuda"),
            "slot": torch.empty(T, k, dtype=torch.int32, device="cuda")}
    y = torch.empty(T, d, dtype=torch_dtype(case), device="cuda")
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    moe.moe_forward(p, dev(inp["x"]), dev(inp["Wg"]) if gate else None,
                    dev(inp["bg"]) if gate and inp["bg"] is not None else None, dev(inp["W1"]), dev(inp["W2"]), y,
                    logits=logits, info=info, ws=ws)
    torch.cuda.synchronize()
    return {"y": host(y), "topk_idx": host(info["topk_idx"]), "slot": host(info["slot"])}


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    case = random_case(i)
    print(f"[random] {case.name}: T={case.T} d={case.d} E={case.E} k={case.k} F={case.F} {case.act} {case.dtype} "
          f"norm={case.normalize} lam={case.lam} cf={case.cf} logits={case.logits}", flush=True)
    inp = moe_inputs.make(case)
    dy = moe_inputs.make_dy(case)
    out = run_train(case, inp, dy)
    fwd = forward_only(case, inp)
    for key in ("y", "topk_idx", "slot"):
        assert np.array_equal(fwd[key], out[key]), f"moe_forward and moe_forward_train differ in {key}"

    # gate logits: within the rigorous bound of the exact sum (fp32 rounding of
    # a value within eps of it)
    if case.logits == "gate":
        z_exact, _ = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
        eps = logit_eps(to_f64(inp["x"]), to_f64(inp["Wg"]), inp["bg"])
        z = out["logits"].astype(np.float64)
        assert np.all(np.abs(z - z_exact) <= 2 * eps + np.spacing(np.abs(z_exact).astype(np.float32))), \
            "gate logits beyond the accumulation bound"
    z32 = out["logits"] if case.logits == "gate" else inp["logits"]

    # routing and dispatch on those logits
    idx, w = oracle.route(z32, case.k, case.normalize, case.lam)
    disp = oracle.dispatch(idx, case.E, oracle.capacity(case.T, case.E, case.k, case.cf))
    assert np.array_equal(out["topk_idx"], idx)
    assert np.max(np.abs(out["topk_w"].astype(np.float64) - w)) <= TOPK_W_ATOL
    assert np.array_equal(out["counts"], disp["counts"])
    assert np.array_equal(out["offsets"], disp["offsets"])
    assert np.array_equal(out["slot"], disp["slot"])
    assert np.array_equal(out["src_token"][:disp["P"]], disp["src_token"])

    # forward output
    tol = TOL[case.dtype]
    y_ref = oracle.forward_tokens(inp["x"], inp["W1"], inp["W2"], idx, w, disp["slot"], act_code(case), case.F)
    errs = {"y": maxrel(out["y"], y_ref)}
    assert errs["y"] <= tol, errs
    dropped = np.all(disp["slot"] < 0, axis=1)
    assert np.all(to_f64(out["y"][dropped]) == 0.0)

    # backward
    ref = oracle.backward(inp["x"], inp.get("Wg"), inp["W1"], inp["W2"], z32, idx, disp["slot"], dy, act_code(case),
                          case.F, case.normalize, case.lam)
    ex_dW1, ex_dx = {}, {}
    if case.act == "relu":
        x64, dy64 = to_f64(inp["x"]), to_f64(dy)
        for t, e, f in relu_unpinned(x64, inp["W1"], idx, disp["slot"], case.F, case.d):
            dh_max = float(np.abs(to_f64(inp["W2"][e, :, f])) @ np.abs(dy64[t]))
            ex_dW1[(e, f)] = ex_dW1.get((e, f), 0.0) + dh_max * np.abs(x64[t])
            ex_dx[(t,)] = ex_dx.get((t,), 0.0) + dh_max * np.abs(to_f64(inp["W1"][e, f]))
    errs["dx"] = within(out["dx"], ref["dx"], tol, ex_dx)
    errs["dW1"] = within(out["dW1"], ref["dW1"], tol, ex_dW1)
    errs["dW2"] = within(out["dW2"], ref["dW2"], tol)
    if case.logits == "gate":
        adz = np.abs(ref["dz"])
        all_rows = ...  # the allowance covers every element
        within(out["dWg"], ref["dWg"], tol, {all_rows: 2.0 ** -7 * (adz.T @ np.abs(to_f64(inp["x"])))})
        within(out["dbg"], ref["dbg"], tol, {all_rows: 2.0 ** -7 * adz.sum(axis=0)})
        errs["dWg"] = maxrel(out["dWg"], ref["dWg"])  # reported; held to the bounds above
        errs["dbg"] = maxrel(out["dbg"], ref["dbg"])
    # experts no kept row reaches have exactly zero weight gradients
    reached = np.zeros(case.E, bool)
    reached[idx[disp["slot"] >= 0]] = True
    assert np.all(out["dW1"][~reached] == 0.0) and np.all(out["dW2"][~reached] == 0.0)
    print(f"  P={disp['P']} dropped={case.T * case.k - disp['P']} " +
          ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


# ------------------------------------------------------------------ FP8 layer
N_FP8_CASES = 12


def random_fp8_case(i):
    """bf16 activations, d and F multiples of 128 (the FP8 layer's limits)."""
    g = np.random.default_rng([7718, i])
    E = int(g.choice([1, 2, 5, 8, 16, 33, 64]))
    return moe_inputs.Case(
        name=f"rand_fp8_{i}",
        T=int(g.choice([1, 3, 64, 129, 300, 777])),
        d=128 * int(g.integers(1, 5)),
        E=E, k=int(g.integers(1, min(E, 8) + 1)),
        F=128 * int(g.integers(1, 5)),
        act=str(g.choice(["relu", "swiglu"])), dtype="bf16",
        seed=7718 * 1000 + i,
        normalize=bool(g.integers(0, 2)),
        lam=float(g.choice([0.5, 1.0, 2.0])),
        cf=float(g.choice([0.0, 0.0, 0.5, 1.0, 1.25])),
        logits=str(g.choice(["gate", "gate", "given"])),
        x_std=1.0, w_std=0.05, wg_std=0.05)


@pytest.mark.parametrize("i", range(N_FP8_CASES))
def test_random_shape_fp8(i):
    case = random_fp8_case(i)
    print(f"[random-fp8] {case.name}: T={case.T} d={case.d} E={case.E} k={case.k} F={case.F} {case.act} "
          f"norm={case.normalize} cf={case.cf} logits={case.logits}", flush=True)
    inp = moe_inputs.make(case)
    W1q, w1s = oracle.quant_weights_fp8(inp["W1"])
    W2q, w2s = oracle.quant_weights_fp8(inp["W2"])
    p = problem_of(case)
    T, E, k, d = case.T, case.E, case.k, case.d
    gate = case.logits == "gate"
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda") if gate else dev(inp["logits"])
    info = {"topk_idx": torch.empty(T, k, dtype=torch.int32, device="cuda"),
            "slot": torch.empty(T, k, dtype=torch.int32, device="cuda")}
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_fp8_workspace_size(p), dtype=torch.uint8, device="cuda")
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()  # noqa: E731
    moe.moe_forward_fp8(p, dev(inp["x"]), dev(inp["Wg"]) if gate else None,
                        dev(inp["bg"]) if gate and inp["bg"] is not None else None, u8(W1q), dev(w1s), u8(W2q),
                        dev(w2s), y, logits=logits, info=info, ws=ws)
    torch.cuda.synchronize()
    z32 = host(logits) if gate else inp["logits"]
    idx, w = oracle.route(z32, k, case.normalize, case.lam)
    disp = oracle.dispatch(idx, E, oracle.capacity(T, E, k, case.cf))
    assert np.array_equal(host(info["topk_idx"]), idx)
    assert np.array_equal(host(info["slot"]), disp["slot"])
    ref = oracle.forward_tokens_fp8(inp["x"], W1q, w1s, W2q, w2s, idx, w, disp["slot"], act_code(case), case.F)
    got = host(y)
    err = maxrel(got, ref)
    # the bf16 layer bar, plus the allowance for E4M3 codes of h that the
    # GPU's bf16 h may round the other way
    allow = fp8_code_allowance(case, inp["x"], W1q, w1s, W2q, w2s, w, disp)
    over = np.abs(to_f64(got) - ref) - (TOL["bf16"] * np.max(np.abs(ref)) + allow)
    assert np.all(over <= 0), f"max-abs-rel {err:.3e}; {float(over.max()):.3e} beyond the bound"
    gone = np.all(disp["slot"] < 0, axis=1)
    assert not got[gone].any()
    print(f"  P={disp['P']} max-abs-rel {err:.2e}", flush=True)
