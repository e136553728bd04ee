"""GPU parity of the layer's backward (moe_forward_train + moe_backward) with
the CPU oracle, through the C ABI.

Bars: routing bit-exact (as in the forward tests); y, dx, dW1, dW2, dWg, dbg
within the layer's max-abs-rel bound (1e-4 fp32, 2e-2 bf16: the GPU stores u,
h, y_perm and the permuted gradients in the layer dtype, the oracle keeps
every intermediate in fp64).  One floating-point decision sits inside the
backward: ReLU's u > 0.  Where the exact u is within the rigorous bound of the
GPU's fp32 accumulation error (tests/_margins.py) either decision is correct;
the dW1 rows and dx rows such an element touches are held to the bar plus the
largest change the other decision could make, every other element to the bar.

Full sizes: dy is nonzero on sampled tokens only, so every gradient depends on
those tokens alone and the oracle runs on that sub-batch (with the full-size
routing and drops), while the GPU runs the whole layer at its full shape in
the benchmark's launch configuration; dx off the sample and dW1/dW2 of
experts the sample does not reach must be exactly zero.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_logit_amd as moe
import moe_inputs
import oracle
from _gpu import TOL, dev, host, maxrel, problem_of, run_train, to_f64, torch_dtype, within
from _margins import relu_unpinned

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SMALL = list(moe_inputs.SMALL)
FULL_SAMPLED = {"fastmoe_txl": 16, "mixtral": 6, "skywork_m_zipf": 6, "many_small": 16, "large_t_bwd": 12}


def act_code(case):
    return oracle.SWIGLU if case.act == "swiglu" else oracle.RELU


def oracle_route(case, inp):
    if case.logits == "gate":
        _ze, z32 = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
    else:
        z32 = inp["logits"]
    idx, w = oracle.route(z32, case.k, case.normalize, case.lam)
    disp = oracle.dispatch(idx, case.E, oracle.capacity(case.T, case.E, case.k, case.cf))
    return z32, idx, w, disp


def check_backward(case, inp, out, dy, tokens=None, aux_coef=0.0, z_coef=0.0):
    z32, idx, w, disp = oracle_route(case, inp)
    assert np.array_equal(out["topk_idx"], idx)
    assert np.array_equal(out["slot"], disp["slot"])
    assert np.array_equal(out["offsets"], disp["offsets"])
    tol = TOL[case.dtype]
    S = np.arange(case.T) if tokens is None else np.asarray(tokens)
    # forward output on the sample
    y_ref = oracle.forward_tokens(inp["x"], inp["W1"], inp["W2"], idx, w, disp["slot"], act_code(case), case.F,
                                  None if tokens is None else S.astype(np.int32))
    errs = {"y": maxrel(out["y"][S], y_ref)}
    assert errs["y"] <= tol, errs
    x_s = inp["x"][S]
    assert tokens is None or not (aux_coef or z_coef), "the balancing losses reach every token"
    ref = oracle.backward(x_s, inp.get("Wg"), inp["W1"], inp["W2"], z32[S], idx[S], disp["slot"][S], dy[S],
                          act_code(case), case.F, case.normalize, case.lam, aux_coef=aux_coef, z_coef=z_coef)
    # ReLU decisions the two sides may take differently, and the most they can
    # change: dh_f <= sum_i |W2[e,i,f] dy_t,i| (gate weight <= 1) moves
    # dW1[e,f,:] by dh_f |x_t| and dx_t by dh_f |W1[e,f,:]|
    ex_dW1, ex_dx = {}, {}
    if case.act == "relu":
        x64 = to_f64(x_s)
        dy64 = to_f64(dy[S])
        for t, e, f in relu_unpinned(x64, inp["W1"], idx[S], disp["slot"][S], case.F, case.d):
            dh_max = float(np.abs(to_f64(inp["W2"][e, :, f])) @ np.abs(dy64[t]))
            ex_dW1[(e, f)] = ex_dW1.get((e, f), 0.0) + dh_max * np.abs(x64[t])
            ex_dx[(t,)] = ex_dx.get((t,), 0.0) + dh_max * np.abs(to_f64(inp["W1"][e, f]))
        if ex_dW1:
            print(f"  {len(ex_dW1)} dW1 rows hold an unpinned ReLU decision", flush=True)
    errs["dx"] = within(out["dx"][S], ref["dx"], tol, ex_dx)
    errs["dW1"] = within(out["dW1"], ref["dW1"], tol, ex_dW1)
    errs["dW2"] = within(out["dW2"], ref["dW2"], tol)
    if case.logits == "gate":
        errs["dWg"] = within(out["dWg"], ref["dWg"], tol)
        errs["dbg"] = within(out["dbg"], ref["dbg"], tol)
    if tokens is not None:
        off = np.ones(case.T, bool)
        off[S] = False
        assert np.all(to_f64(out["dx"][off]) == 0.0)
        reached = np.zeros(case.E, bool)
        reached[idx[S][disp["slot"][S] >= 0]] = True
        assert np.all(out["dW1"][~reached] == 0.0) and np.all(out["dW2"][~reached] == 0.0)
    return errs


@pytest.mark.parametrize("name", SMALL)
def test_backward_small(name):
    case = moe_inputs.get(name)
    print(f"[backward] {name}", flush=True)
    inp = moe_inputs.make(case)
    dy = moe_inputs.make_dy(case)
    out = run_train(case, inp, dy)
    errs = check_backward(case, inp, out, dy)
    print("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


@pytest.mark.parametrize("E", [8, 16])
def test_backward_split_tail_tiles(E):
    """The training step on the 128 x 128 (E = 8: 128 rows per expert) and
    64 x 256 (E = 16: 64 rows) tiles, whose waves hold one 32-column block,
    with the K-split tail in every GEMM whose K reaches 2048: the
    up-projection (K = d), the activation-backward GEMM (K = d) and the
    input-gradient GEMM (K = 2F).  Capacity factor 1 keeps each expert within
    one m-tile, so few enough tiles remain for their last round to split."""
    case = moe_inputs.get("mixtral_s").with_(name=f"bsplit_E{E}", T=512, d=2048, F=1024, E=E, cf=1.0, bias="none")
    print(f"[backward split tail] {case.name}", flush=True)
    inp = moe_inputs.make(case)
    dy = moe_inputs.make_dy(case)
    out = run_train(case, inp, dy)
    errs = check_backward(case, inp, out, dy)
    print("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


def sample(case, inp, n):
    g = np.random.default_rng(case.seed + 77)
    picks = {0, case.T - 1}
    picks.update(g.choice(case.T, size=n, replace=False).tolist())
    z32, idx, _w, disp = oracle_route(case, inp)
    dropped = np.nonzero(np.any(disp["slot"] < 0, axis=1))[0]
    picks.update(dropped[:2].tolist())
    return np.array(sorted(picks), np.int64)


@pytest.mark.parametrize("name", list(FULL_SAMPLED))
def test_backward_full_size_sampled(name):
    case = moe_inputs.get(name)
    print(f"[backward-full] {name}", flush=True)
    inp = moe_inputs.make(case)
    toks = sample(case, inp, FULL_SAMPLED[name])
    dy = moe_inputs.make_dy(case, tokens=toks)
    out = run_train(case, inp, dy)
    errs = check_backward(case, inp, out, dy, tokens=toks)
    print(f"  {len(toks)} tokens: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


@pytest.mark.parametrize("name", ["skywork_m_zipf_s", "many_small_s"])
def test_backward_deterministic_and_workspace_independent(name):
    case = moe_inputs.get(name)
    print(f"[backward-det] {name}", flush=True)
    inp = moe_inputs.make(case)
    dy = moe_inputs.make_dy(case)
    a = run_train(case, inp, dy, ws_fill=0)
    b = run_train(case, inp, dy, ws_fill=0xFF)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("kind", ["T0", "T1", "E_equals_k", "k1_norm", "single_expert", "heavy_drop", "all_to_one",
                                  "constant_norm", "fp32_swiglu_norm", "fp32_relu_given", "shared_expert_e1"])
def test_backward_edges(kind):
    print(f"[backward-edge] {kind}", flush=True)
    base = moe_inputs.get("mixtral_s").with_(bias="none")
    if kind == "T0":
        case = base.with_(name="bedge_T0", T=0)
    elif kind == "T1":
        case = base.with_(name="bedge_T1", T=1)
    elif kind == "E_equals_k":
        case = base.with_(name="bedge_Ek", E=2, k=2, act="relu")
    elif kind == "k1_norm":
        case = base.with_(name="bedge_k1", k=1, normalize=True, lam=2.0)
    elif kind == "single_expert":
        case = base.with_(name="bedge_E1", E=1, k=1)
    elif kind == "heavy_drop":
        case = base.with_(name="bedge_drop", cf=0.25, normalize=True, act="relu")
    elif kind == "all_to_one":
        case = base.with_(name="bedge_one", cf=0.5)
    elif kind == "constant_norm":
        case = base.with_(name="bedge_const", normalize=True, T=64)
    elif kind == "fp32_swiglu_norm":
        case = base.with_(name="bedge_f32", dtype="f32", x_std=0.5, normalize=True, lam=2.0, cf=1.0, T=300)
    elif kind == "shared_expert_e1":
        # a shared expert is the layer with one expert, top-1 and given logits
        # (the softmax of a single logit is exactly 1): its training step
        case = base.with_(name="bedge_shared", E=1, k=1, logits="given")
    else:
        case = moe_inputs.get("tiny_fp32").with_(name="bedge_f32_given", logits="given", E=6, k=3, T=200, cf=1.0)
    inp = moe_inputs.make(case)
    if kind in ("all_to_one", "constant_norm"):
        # every token's logits equal the bias: favour experts 5 then 2, or all equal
        inp["Wg"] = np.zeros_like(inp["Wg"])
        bg = np.zeros(case.E, np.float32)
        if kind == "all_to_one":
            bg[5], bg[2] = 2.0, 1.0
        inp["bg"] = bg
    dy = moe_inputs.make_dy(case)
    out = run_train(case, inp, dy)
    if case.T == 0:
        assert np.all(out["dW1"] == 0.0) and np.all(out["dW2"] == 0.0)
        assert np.all(out["dWg"] == 0.0) and np.all(out["dbg"] == 0.0)
        return
    errs = check_backward(case, inp, out, dy)
    if kind == "shared_expert_e1":  # the same output as the oracle's shared expert
        ys = oracle.shared_expert(inp["x"], inp["W1"][0], inp["W2"][0], act_code(case), case.F)
        assert maxrel(out["y"], ys) <= TOL[case.dtype]
    if kind == "constant_norm":  # sigma == 0: no gradient reaches the logits
        assert np.all(out["dWg"] == 0.0) and np.all(out["dbg"] == 0.0)
    print("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


@pytest.mark.parametrize("name,dy_zero", [("mixtral_s", False), ("skywork_m_zipf_s", False),
                                          ("skywork_m_zipf_s", True)])
def test_backward_balancing_losses(name, dy_zero):
    """The auxiliary loss and Z-loss gradients (coefficients 0.3 and 0.05); with
    dy = 0 they are the only source, so the expert weight gradients are 0."""
    case = moe_inputs.get(name)
    print(f"[backward-losses] {name} dy_zero={dy_zero}", flush=True)
    inp = moe_inputs.make(case)
    dy = moe_inputs.make_dy(case)
    if dy_zero:
        dy = np.zeros_like(dy)
    out = run_train(case, inp, dy, aux_coef=0.3, z_coef=0.05)
    errs = check_backward(case, inp, out, dy, aux_coef=0.3, z_coef=0.05)
    if dy_zero:
        assert np.all(out["dW1"] == 0.0) and np.all(out["dW2"] == 0.0)
        assert np.any(out["dWg"] != 0.0)
    print("  " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)

