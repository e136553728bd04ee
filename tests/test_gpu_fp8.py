"""GPU parity of the FP8 (E4M3) expert path with the CPU oracle, through the C ABI.

Bars:
  * quantisation: codes and scales bit-exact (a power-of-two scale makes the
    value to round exact on both sides, and both round to nearest-even);
  * each FP8 GEMM alone, on the oracle's codes: the products of E4M3 values
    are exact in fp32, so the GPU differs only by fp32 accumulation order and
    the bf16 store of its output: the bf16 bar, max-abs-rel <= 2e-2;
  * the whole FP8 layer: besides those roundings, the GPU quantises its own
    bf16 h while the oracle quantises the exact h; where the two straddle an
    E4M3 rounding boundary (the bf16 store moves h by <= 2^-9 relative, about
    1/32 of an E4M3 step) a code differs by one step (<= 2^-3 relative) and
    moves each output by that step times one weight.  Each output element is
    held to the bf16 bar (2e-2 of max|y|) plus the largest change such flips
    can make to it, computed from the oracle's exact h (tests/_fp8_bound.py);
    where no code of h can straddle, that is the plain bf16 bar.  Routing
    (bf16 gate) is bit-exact.
Inputs come from the seeded generator and the oracle (including every code
and scale fed to the GPU GEMMs), never from the GPU.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_logit_amd as moe
import moe_inputs
import oracle
from _gpu import TOL, dev, host, maxrel, problem_of, to_f64
from _fp8_bound import fp8_code_allowance
import _tiles

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

RNG = np.random.default_rng(31337)
TOL_GEMM = 2e-2

# Small FP8 workloads (d and F multiples of 128), ragged segments and drops.
FP8_SMALL = {
    # name: (base case, overrides)
    "mixtral_fp8_s": ("mixtral_s", dict(d=256, F=384)),
    "txl_fp8_s": ("fastmoe_txl_s", dict()),
    "skywork_fp8_s": ("skywork_m_s", dict(d=384, F=384)),
    "skywork_zipf_fp8_s": ("skywork_m_zipf_s", dict(d=384, F=384)),
    "many_small_fp8_s": ("many_small_s", dict(F=128)),
    # the 256 x 256 FP8 tile, every output checked
    "mixtral_fp8_m": ("mixtral_m", dict()),
    "mixtral_fp8_m_cap": ("mixtral_m_cap", dict()),
}


def fp8_case(name):
    base, over = FP8_SMALL[name]
    return moe_inputs.get(base).with_(**over)


def fp8_bias_override(case):
    """A Zipf-skewed FP8 variant whose d differs from its base case reuses the
    base case's stored gate bias (the skew stays, its exact shares do not)."""
    for name, (base, over) in FP8_SMALL.items():
        b = moe_inputs.get(base)
        if case.name == b.name and case.bias == "zipf" and case.d != b.d:
            return moe_inputs.zipf_bias(b)
    return None


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


_cache = {}


def fp8_inputs(case):
    key = (case.name, case.d, case.F)
    if key not in _cache:
        _cache.clear()
        inp = moe_inputs.make(case, bias_override=fp8_bias_override(case))
        W1q, w1s = oracle.quant_weights_fp8(inp["W1"])
        W2q, w2s = oracle.quant_weights_fp8(inp["W2"])
        inp.update(W1q=W1q, w1s=w1s, W2q=W2q, w2s=w2s)
        _cache[key] = inp
    return _cache[key]


def routing(case, inp):
    if case.logits == "gate":
        _ze, z32 = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
    else:
        z32 = inp["logits"]
    idx, w = oracle.route(z32, case.k, case.normalize, case.lam)
    disp = oracle.dispatch(idx, case.E, oracle.capacity(case.T, case.E, case.k, case.cf))
    return idx, w, disp


# ------------------------------------------------------------------ quantisation
@pytest.mark.parametrize("dtype,K", [("bf16", 384), ("f32", 384), ("bf16", 4096), ("bf16", 14336),
                                     ("bf16", 16384), ("bf16", 20480), ("f32", 14336)])
def test_quantize_fp8_bit_exact(dtype, K):
    # bf16 rows up to 16384 values take the register-resident kernel, longer
    # rows and fp32 rows the two-pass one
    print(f"[fp8-quant] {dtype} K={K}", flush=True)
    R = 517 if K <= 4096 else 67
    v = (RNG.standard_normal((R, K)) * np.exp(RNG.uniform(-20, 20, (R, 1)))).astype(np.float32)
    v[0] = 0.0                                    # zero row: scale 1, codes 0
    v[1] = 448.0 * 2.0 ** -3                      # exactly at a scale boundary
    v[2, :] = 1e-3
    v[2, 7] = -448.0 * 2.0 ** 5 * 1.0000001       # just above a boundary
    v[3] = np.float32(2.0 ** -120) * RNG.standard_normal(K).astype(np.float32)  # tiny row
    v[4, ::2] = -0.0
    src = moe_inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v
    codes_ref, scales_ref = oracle.quant_rows_fp8(src)
    t = dev(src)
    codes = torch.empty(R, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(R, dtype=torch.float32, device="cuda")
    moe.moe_quantize_fp8(t, codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(host(scales), scales_ref)
    assert np.array_equal(host(codes), codes_ref)


# ------------------------------------------------------------------ FP8 GEMMs
@pytest.mark.parametrize("name", list(FP8_SMALL))
def test_expert_up_and_down_fp8(name):
    case = fp8_case(name)
    print(f"[fp8-ffn] {name} T={case.T} d={case.d} F={case.F}", flush=True)
    inp = fp8_inputs(case)
    p = problem_of(case)
    idx, w, disp = routing(case, inp)
    P, Tk = disp["P"], case.T * case.k
    act = oracle.SWIGLU if case.act == "swiglu" else oracle.RELU
    xq, xs = oracle.quant_rows_fp8(inp["x"])
    src = disp["src_token"]
    _y, ref_h = oracle.ffn_rows_fp8(xq[src], xs[src], disp["offsets"], inp["W1q"], inp["w1s"], inp["W2q"],
                                    inp["w2s"], act, case.F, want_h=True)
    off_d = dev(disp["offsets"])
    src_d = torch.full((Tk,), -1, dtype=torch.int32, device="cuda")
    src_d[:P] = dev(src)
    W1q, w1s, W2q, w2s = u8(inp["W1q"]), dev(inp["w1s"]), u8(inp["W2q"]), dev(inp["w2s"])
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    # gathered through src_token, with the K-split workspace
    h = torch.zeros(Tk, case.F, dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_up_fp8(p, u8(xq), dev(xs), src_d, off_d, W1q, w1s, h, ws=ws)
    # the same rows as a permuted copy, without the workspace
    xpq = np.zeros((Tk, case.d), np.uint8)
    xpq[:P] = xq[src]
    xps = np.ones(Tk, np.float32)
    xps[:P] = xs[src]
    h2 = torch.zeros_like(h)
    moe.moe_expert_up_fp8(p, u8(xpq), dev(xps), None, off_d, W1q, w1s, h2)
    torch.cuda.synchronize()
    assert maxrel(host(h)[:P], ref_h) <= TOL_GEMM
    assert maxrel(host(h2)[:P], ref_h) <= TOL_GEMM
    # down on quantised synthetic hidden rows
    hq, hs = oracle.quant_rows_fp8(np.abs(RNG.standard_normal((max(P, 1), case.F))).astype(np.float32))
    hq_d = torch.zeros(Tk, case.F, dtype=torch.uint8, device="cuda")
    hq_d[:P] = u8(hq[:P])
    hs_d = torch.ones(Tk, dtype=torch.float32, device="cuda")
    hs_d[:P] = dev(hs[:P])
    yp = torch.zeros(Tk, case.d, dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_down_fp8(p, hq_d, hs_d, off_d, W2q, w2s, yp, ws=ws)
    torch.cuda.synchronize()
    ref_y = oracle.down_rows_fp8(hq[:max(P, 1)], hs[:max(P, 1)], disp["offsets"], inp["W2q"], inp["w2s"])
    assert maxrel(host(yp)[:P], ref_y[:P]) <= TOL_GEMM


# Segment layouts that make the last tile round split along K (one per tile
# configuration), FP8 weights.
FP8_SPLIT = {
    "large": ("swiglu", 1024, 2048, 4, 2, 1536, [700, 300, 512, 536]),
    "medium": ("relu", 512, 2048, 4, 2, 1024, [300, 0, 257, 300]),
    "small": ("relu", 512, 2048, 16, 2, 512, [64] * 14 + [1, 63]),
}


@pytest.mark.parametrize("name", list(FP8_SPLIT))
def test_fp8_split_tail(name):
    act, T, d, E, k, F, seg = FP8_SPLIT[name]
    print(f"[fp8-split] {name}", flush=True)
    p = moe.problem(T, d, E, k, F, act=act, dtype="bf16")
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    P = int(offsets[-1])
    n1 = 2 * F if act == "swiglu" else F
    rng = np.random.default_rng(77 + len(name))
    xq, xs = oracle.quant_rows_fp8(rng.standard_normal((P, d)).astype(np.float32))
    W1q, w1s = oracle.quant_weights_fp8((rng.standard_normal((E, n1, d)) / np.sqrt(d)).astype(np.float32))
    W2q, w2s = oracle.quant_weights_fp8((rng.standard_normal((E, d, F)) / np.sqrt(F)).astype(np.float32))
    hq, hs = oracle.quant_rows_fp8(np.abs(rng.standard_normal((P, F))).astype(np.float32))
    actc = oracle.SWIGLU if act == "swiglu" else oracle.RELU
    _y, ref_h = oracle.ffn_rows_fp8(xq, xs, offsets, W1q, w1s, W2q, w2s, actc, F, want_h=True)
    ref_y = oracle.down_rows_fp8(hq, hs, offsets, W2q, w2s)
    Tk = T * k
    pad = lambda a, n, fill: np.concatenate([a, np.full((n - a.shape[0],) + a.shape[1:], fill, a.dtype)])
    xq_d, xs_d = u8(pad(xq, Tk, 0)), dev(pad(xs, Tk, 1.0))
    hq_d, hs_d = u8(pad(hq, Tk, 0)), dev(pad(hs, Tk, 1.0))
    off_d = dev(offsets)
    ws = torch.full((moe.moe_workspace_size(p),), 0xFF, dtype=torch.uint8, device="cuda")
    h = torch.zeros(Tk, F, dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_up_fp8(p, xq_d, xs_d, None, off_d, u8(W1q), dev(w1s), h, ws=ws)
    torch.cuda.synchronize()
    assert int((ws != 0xFF).sum()) > 0, "the K split did not run"
    yp = torch.zeros(Tk, d, dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_down_fp8(p, hq_d, hs_d, off_d, u8(W2q), dev(w2s), yp, ws=ws)
    torch.cuda.synchronize()
    assert maxrel(host(h)[:P], ref_h) <= TOL_GEMM
    assert maxrel(host(yp)[:P], ref_y) <= TOL_GEMM
    assert not host(h)[P:].any() and not host(yp)[P:].any()


# ------------------------------------------------------------------ whole FP8 layer
def run_forward_fp8(case, inp):
    p = problem_of(case)
    T, E, k, d = case.T, case.E, case.k, case.d
    x = dev(inp["x"])
    Wg = dev(inp["Wg"]) if inp["Wg"] is not None else None
    bg = dev(inp["bg"]) if inp["bg"] is not None else None
    logits = dev(inp["logits"]) if case.logits == "given" else torch.empty(T, E, dtype=torch.float32, device="cuda")
    info = {"topk_idx": torch.empty(T, k, dtype=torch.int32, device="cuda"),
            "slot": torch.empty(T, k, dtype=torch.int32, device="cuda")}
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_fp8_workspace_size(p), dtype=torch.uint8, device="cuda")
    moe.moe_forward_fp8(p, x, Wg, bg, u8(inp["W1q"]), dev(inp["w1s"]), u8(inp["W2q"]), dev(inp["w2s"]), y,
                        logits=logits, info=info, ws=ws)
    torch.cuda.synchronize()
    return host(y), host(info["topk_idx"]), host(info["slot"])


@pytest.mark.parametrize("name", list(FP8_SMALL))
def test_forward_fp8(name):
    case = fp8_case(name)
    print(f"[fp8-layer] {name}", flush=True)
    inp = fp8_inputs(case)
    idx, w, disp = routing(case, inp)
    y, gidx, gslot = run_forward_fp8(case, inp)
    assert np.array_equal(gidx, idx) and np.array_equal(gslot, disp["slot"])
    act = oracle.SWIGLU if case.act == "swiglu" else oracle.RELU
    ref = oracle.forward_tokens_fp8(inp["x"], inp["W1q"], inp["w1s"], inp["W2q"], inp["w2s"], idx, w,
                                    disp["slot"], act, case.F)
    check_fp8_layer(case, inp, w, disp, y, ref)
    gone = np.all(disp["slot"] < 0, axis=1)
    assert not y[gone].any()


def check_fp8_layer(case, inp, w, disp, got, ref, tokens=None):
    """Every element within the bf16 bar plus its derived allowance for E4M3
    codes of h that the GPU's bf16 h may round the other way."""
    allow = fp8_code_allowance(case, inp["x"], inp["W1q"], inp["w1s"], inp["W2q"], inp["w2s"], w, disp, tokens)
    over = np.abs(to_f64(got) - ref) - (TOL["bf16"] * np.max(np.abs(ref)) + allow)
    err = maxrel(got, ref)
    assert np.all(over <= 0), f"max-abs-rel {err:.3e}; {float(over.max()):.3e} beyond the bound"
    print(f"  max-abs-rel {err:.2e}, mean allowance {float(allow.mean() / max(np.max(np.abs(ref)), 1e-30)):.2e} "
          f"of max|y|", flush=True)


def test_forward_fp8_full_size_sampled():
    """The Mixtral-shaped layer with FP8 experts, checked on sampled tokens."""
    case = moe_inputs.get("mixtral")
    print("[fp8-layer-full] mixtral", flush=True)
    inp = fp8_inputs(case)
    idx, w, disp = routing(case, inp)
    y, gidx, gslot = run_forward_fp8(case, inp)
    assert np.array_equal(gidx, idx) and np.array_equal(gslot, disp["slot"])
    # tokens whose rows reach every m-tile of every expert and every row of
    # the smallest tile that the last round of each GEMM splits along K
    G = torch.cuda.get_device_properties(0).multi_processor_count
    toks = _tiles.covering_tokens(disp["offsets"], disp["src_token"], [(case.F + 127) // 128, (case.d + 255) // 256],
                                  G, extra=np.random.default_rng(5).choice(case.T, 12, replace=False))
    ref = oracle.forward_tokens_fp8(inp["x"], inp["W1q"], inp["w1s"], inp["W2q"], inp["w2s"], idx, w,
                                    disp["slot"], oracle.SWIGLU, case.F, tokens=toks)
    check_fp8_layer(case, inp, w, disp, y[toks], ref, tokens=toks)
