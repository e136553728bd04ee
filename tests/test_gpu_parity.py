"""GPU parity of the HIP path with the CPU oracle, through the C ABI.

Bars: routing (expert ids and their order), counts, offsets, slots, source
tokens and permuted rows are compared bit for bit; floating outputs within
max|gpu - oracle| / max|oracle| <= 1e-4 (fp32) or 2e-2 (bf16); stored gate
weights within 1e-5 absolute.  Every input comes from the seeded generator or
from the oracle, never from the GPU.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_logit_amd as moe
import moe_inputs
import oracle
from _gpu import TOL, TOPK_W_ATOL, dev, host, maxrel, problem_of, run_forward, to_f64, torch_dtype
from _margins import exact_sum_certified, logit_eps, unstable_keys
import _tiles

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SMALL = list(moe_inputs.SMALL)
FULL = list(moe_inputs.FULL)
GATE_SMALL = [n for n in SMALL if moe_inputs.get(n).logits == "gate"]
GATE_FULL = [n for n in FULL if moe_inputs.get(n).logits == "gate"]

_cache = {}


def inputs(name, weights=True):
    key = (name, weights)
    if key not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        _cache[key] = moe_inputs.make(name, weights=weights)
    return _cache[key]


def act_code(case):
    return oracle.SWIGLU if case.act == "swiglu" else oracle.RELU


def oracle_route(case, inp):
    """Oracle gate (or given logits) and routing of a case."""
    if case.logits == "gate":
        z_exact, z32 = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
    else:
        z_exact, z32 = None, inp["logits"]
    idx, w = oracle.route(z32, case.k, case.normalize, case.lam)
    C = oracle.capacity(case.T, case.E, case.k, case.cf)
    disp = oracle.dispatch(idx, case.E, C)
    return z_exact, z32, idx, w, disp


# ------------------------------------------------------------------ gate GEMM
@pytest.mark.parametrize("name", GATE_SMALL + GATE_FULL)
def test_gate_logits(name):
    case = moe_inputs.get(name)
    inp = inputs(name, weights=False)
    print(f"[gate] {name}", flush=True)
    p = problem_of(case)
    logits = torch.empty(case.T, case.E, dtype=torch.float32, device="cuda")
    idx = torch.empty(case.T, case.k, dtype=torch.int32, device="cuda")
    w = torch.empty(case.T, case.k, dtype=torch.float32, device="cuda")
    moe.moe_route(p, dev(inp["x"]), dev(inp["Wg"]), dev(inp["bg"]) if inp["bg"] is not None else None,
                  logits, idx, w)
    torch.cuda.synchronize()
    z_exact, z32 = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
    x64, w64 = oracle.to_f64(inp["x"]), oracle.to_f64(inp["Wg"])
    eps = logit_eps(x64, w64, inp["bg"])
    free = unstable_keys(z_exact, eps) & ~exact_sum_certified(x64, w64, inp["bg"], 7 if case.dtype == "bf16" else 23)
    got = host(logits)
    # every pinned key is bit-identical; an unpinned one is within one fp32 step
    assert np.array_equal(got[~free], z32[~free])
    if free.any():
        assert np.all(np.abs(got[free].astype(np.float64) - z_exact[free]) <= np.spacing(np.abs(z32[free])))
    # routing from the GPU's own logits equals the oracle's
    oidx, ow = oracle.route(z32, case.k, case.normalize, case.lam)
    assert np.array_equal(host(idx), oidx)
    assert np.max(np.abs(host(w) - ow)) <= TOPK_W_ATOL


# Gate and router: every column-tile count (E up to 16, 32, 48, 64) and the
# separate kernels beyond 64 experts; T = 37 leaves a partial 16-token block
# and d = 192 gives some wavefronts no 32-element block of the model dimension.
@pytest.mark.parametrize("E", [1, 2, 15, 16, 17, 32, 33, 48, 49, 64, 65])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_route_expert_counts(E, dtype):
    T, d = 37, 192
    print(f"[gate-route] E={E} {dtype}", flush=True)
    rng = np.random.default_rng(9000 + 10 * E + (dtype == "f32"))
    x = moe_inputs._cast(rng.standard_normal((T, d)).astype(np.float32), dtype)
    Wg = moe_inputs._cast((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32), dtype)
    bg = (rng.standard_normal(E) * 0.1).astype(np.float32)
    z_exact, z32 = oracle.gate_logits(x, Wg, bg)
    x64, w64 = oracle.to_f64(x), oracle.to_f64(Wg)
    free = unstable_keys(z_exact, logit_eps(x64, w64, bg)) & ~exact_sum_certified(
        x64, w64, bg, 7 if dtype == "bf16" else 23)
    for k, normalize, lam in [(min(2, E), False, 1.0), (min(E, 8), True, 2.0), (1, True, 0.5)]:
        p = moe.problem(T, d, E, k, 64, normalize=normalize, lam=lam, dtype=dtype)
        logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, dtype=torch.float32, device="cuda")
        moe.moe_route(p, dev(x), dev(Wg), dev(bg), logits, idx, w)
        torch.cuda.synchronize()
        got = host(logits)
        assert np.array_equal(got[~free], z32[~free])
        if free.any():
            assert np.all(np.abs(got[free].astype(np.float64) - z_exact[free]) <= np.spacing(np.abs(z32[free])))
        # routing decided on the GPU's own logits, as the oracle decides it
        oi, ow = oracle.route(got, k, normalize, lam)
        assert np.array_equal(host(idx), oi), (k, normalize)
        assert np.max(np.abs(host(w).astype(np.float64) - ow)) <= TOPK_W_ATOL


# ------------------------------------------------------------------ router on given logits
def route_gpu(z32, k, normalize=False, lam=1.0):
    T, E = z32.shape
    p = moe.problem(T, 64, E, k, 64, normalize=normalize, lam=lam)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_route(p, None, None, None, dev(np.ascontiguousarray(z32, np.float32)), idx, w)
    torch.cuda.synchronize()
    return host(idx), host(w)


def check_route(z32, k, normalize=False, lam=1.0):
    gi, gw = route_gpu(z32, k, normalize, lam)
    oi, ow = oracle.route(z32, k, normalize, lam)
    assert np.array_equal(gi, oi)
    assert np.max(np.abs(gw.astype(np.float64) - ow)) <= TOPK_W_ATOL


@pytest.mark.parametrize("name", SMALL + FULL)
def test_route_given_logits(name):
    case = moe_inputs.get(name)
    inp = inputs(name, weights=False)
    print(f"[route] {name}", flush=True)
    z32 = inp["logits"] if case.logits == "given" else oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])[1]
    check_route(z32, case.k, case.normalize, case.lam)


RNG = np.random.default_rng(777)


@pytest.mark.parametrize("kind", ["ties", "signed_zero", "constant_norm", "large", "tiny", "one_token",
                                  "k_equals_E", "single_expert", "max_experts", "max_k"])
def test_route_edges(kind):
    print(f"[route-edge] {kind}", flush=True)
    if kind == "ties":
        z = RNG.choice(np.array([0.0, 1.0, 2.0], np.float32), size=(300, 12))
        for k in (1, 2, 5):
            check_route(z, k)
            check_route(z, k, True, 1.0)
    elif kind == "signed_zero":
        z = RNG.choice(np.array([-0.0, 0.0, -1.0], np.float32), size=(200, 8))
        check_route(z, 3)
    elif kind == "constant_norm":
        z = np.full((64, 16), 0.3, np.float32)
        check_route(z, 2, True, 1.0)
    elif kind == "large":
        z = (RNG.standard_normal((128, 64)) * 1e4).astype(np.float32)
        check_route(z, 2)
        check_route(z, 4, True, 2.5)
    elif kind == "tiny":
        z = (RNG.standard_normal((128, 64)) * 1e-38).astype(np.float32)   # subnormals
        check_route(z, 2)
    elif kind == "one_token":
        check_route(RNG.standard_normal((1, 16)).astype(np.float32), 2)
    elif kind == "k_equals_E":
        check_route(RNG.standard_normal((100, 6)).astype(np.float32), 6, True, 1.0)
    elif kind == "single_expert":
        check_route(RNG.standard_normal((50, 1)).astype(np.float32), 1)
    elif kind == "max_experts":
        z = RNG.standard_normal((300, 1024)).astype(np.float32)
        check_route(z, 8)
        check_route(z, 2, True, 1.0)
    elif kind == "max_k":
        check_route(RNG.standard_normal((257, 40)).astype(np.float32), 8, True, 0.5)


# ------------------------------------------------------------------ permutation
def permute_gpu(case, idx, x):
    p = problem_of(case)
    T, E, k, d = case.T, case.E, case.k, case.d
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    slot = torch.empty(T, k, dtype=torch.int32, device="cuda")
    src = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    xp = torch.zeros(T * k, d, dtype=torch_dtype(case), device="cuda")
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    moe.moe_permute(p, dev(idx), dev(x), counts, offsets, slot, src, xp, ws)
    torch.cuda.synchronize()
    return host(counts), host(offsets), host(slot), host(src), host(xp)


def check_permute(case, idx, x):
    C = oracle.capacity(case.T, case.E, case.k, case.cf)
    o = oracle.dispatch(idx, case.E, C)
    counts, offsets, slot, src, xp = permute_gpu(case, idx, x)
    P = o["P"]
    assert np.array_equal(counts, o["counts"])
    assert np.array_equal(offsets, o["offsets"])
    assert np.array_equal(slot, o["slot"])
    assert np.array_equal(src[:P], o["src_token"])
    assert np.array_equal(xp[:P], x[o["src_token"]])
    return o


@pytest.mark.parametrize("name", SMALL + FULL)
def test_permute(name):
    case = moe_inputs.get(name)
    inp = inputs(name, weights=False)
    print(f"[permute] {name}", flush=True)
    _ze, _z32, idx, _w, _d = oracle_route(case, inp)
    check_permute(case, idx, inp["x"])


@pytest.mark.parametrize("kind", ["heavy_drop", "one_expert", "empty_experts", "max_experts", "k8_capacity",
                                  "ragged_T", "scan_in_scatter_limit", "scan_launched", "cf_not_dyadic"])
def test_permute_edges(kind):
    print(f"[permute-edge] {kind}", flush=True)
    base = moe_inputs.get("mixtral_s")
    if kind == "cf_not_dyadic":
        # fp32(0.3) * 600 * 2 / 8 = 45.0000018: the capacity is 46, one above
        # the decimal product; skewed logits make the clip bite on most experts
        case = base.with_(cf=0.3)
        assert oracle.capacity(case.T, case.E, case.k, case.cf) == 46 == moe.moe_capacity(problem_of(case))
        idx = oracle.route(RNG.standard_normal((case.T, case.E)).astype(np.float32) + np.linspace(
            1, 0, case.E, dtype=np.float32), case.k)[0]
        o = check_permute(case, idx, moe_inputs.f32_to_bf16_bits(
            RNG.standard_normal((case.T, case.d)).astype(np.float32)))
        assert int(np.sum(o["counts"] > 46)) >= 4 and o["P"] < case.T * case.k
        return
    if kind == "heavy_drop":
        case = base.with_(cf=0.25)
        idx = oracle.route(RNG.standard_normal((case.T, case.E)).astype(np.float32) + np.linspace(2, 0, case.E,
                           dtype=np.float32), case.k)[0]
    elif kind == "one_expert":
        case = base.with_(k=1, cf=0.5)
        idx = np.zeros((case.T, 1), np.int32)
    elif kind == "empty_experts":
        case = base.with_(E=32)
        idx = np.stack([RNG.choice(np.array([3, 17, 30]), size=2, replace=False) for _ in range(case.T)]).astype(
            np.int32)
    elif kind == "max_experts":
        case = base.with_(E=1024, T=3000, k=4)
        idx = oracle.route(RNG.standard_normal((case.T, case.E)).astype(np.float32), case.k)[0]
    elif kind == "k8_capacity":
        case = base.with_(E=40, k=8, cf=1.0, T=777)
        idx = oracle.route(RNG.standard_normal((case.T, case.E)).astype(np.float32) * np.linspace(
            1, 3, 40, dtype=np.float32), case.k)[0]
    elif kind in ("scan_in_scatter_limit", "scan_launched"):
        # 256-token chunks x 1024 experts: 64 chunks is the most for which the
        # scatter kernel scans the chunk counts itself; 65 launches the scan
        case = base.with_(E=1024, k=2, cf=1.0, T=16384 if kind == "scan_in_scatter_limit" else 16385)
        idx = oracle.route(RNG.standard_normal((case.T, case.E)).astype(np.float32) * np.linspace(
            1, 2, case.E, dtype=np.float32), case.k)[0]
    else:
        case = base.with_(T=257)
        idx = oracle.route(RNG.standard_normal((case.T, case.E)).astype(np.float32), case.k)[0]
    x = moe_inputs.f32_to_bf16_bits(RNG.standard_normal((case.T, case.d)).astype(np.float32))
    check_permute(case, idx, x)


# ------------------------------------------------------------------ expert FFN
def permuted_inputs(case, inp):
    _ze, _z32, idx, w, disp = oracle_route(case, inp)
    xp = inp["x"][disp["src_token"]]
    return idx, w, disp, xp


@pytest.mark.parametrize("name", SMALL)
def test_expert_up_and_down(name):
    case = moe_inputs.get(name)
    inp = inputs(name)
    print(f"[ffn] {name}", flush=True)
    p = problem_of(case)
    _idx, _w, disp, xp = permuted_inputs(case, inp)
    P = disp["P"]
    rows_cap = case.T * case.k
    dt = torch_dtype(case)
    xp_d = torch.zeros(rows_cap, case.d, dtype=dt, device="cuda")
    xp_d[:P] = dev(xp)
    off_d = dev(disp["offsets"])
    src_d = torch.full((rows_cap,), -1, dtype=torch.int32, device="cuda")
    src_d[:P] = dev(disp["src_token"])
    W1 = dev(inp["W1"])
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    h = torch.zeros(rows_cap, case.F, dtype=dt, device="cuda")
    moe.moe_expert_up(p, xp_d, None, off_d, W1, h)
    # the same rows gathered from x through src_token: the same tiles in the
    # same order, so bit-identical
    hg = torch.zeros(rows_cap, case.F, dtype=dt, device="cuda")
    moe.moe_expert_up(p, dev(inp["x"]), src_d, off_d, W1, hg, ws=ws)
    hw = torch.zeros(rows_cap, case.F, dtype=dt, device="cuda")
    moe.moe_expert_up(p, xp_d, None, off_d, W1, hw, ws=ws)
    torch.cuda.synchronize()
    ref_y, ref_h = oracle.ffn_rows(xp, disp["offsets"], inp["W1"], inp["W2"], act_code(case), case.F, want_h=True)
    assert maxrel(host(h)[:P], ref_h) <= TOL[case.dtype]
    assert maxrel(host(hw)[:P], ref_h) <= TOL[case.dtype]
    assert np.array_equal(host(hg)[:P], host(hw)[:P])
    # down on synthetic hidden rows
    hs = moe_inputs._cast(RNG.standard_normal((P, case.F)).astype(np.float32), case.dtype)
    hs_d = torch.zeros(rows_cap, case.F, dtype=dt, device="cuda")
    hs_d[:P] = dev(hs)
    yp = torch.zeros(rows_cap, case.d, dtype=dt, device="cuda")
    moe.moe_expert_down(p, hs_d, off_d, dev(inp["W2"]), yp, ws=ws)
    torch.cuda.synchronize()
    assert maxrel(host(yp)[:P], oracle.down_rows(hs, disp["offsets"], inp["W2"])) <= TOL[case.dtype]
    # both layers through moe_grouped_ffn (h in the workspace)
    yp2 = torch.zeros(rows_cap, case.d, dtype=dt, device="cuda")
    moe.moe_grouped_ffn(p, xp_d, off_d, W1, dev(inp["W2"]), yp2, ws)
    torch.cuda.synchronize()
    assert maxrel(host(yp2)[:P], ref_y) <= TOL[case.dtype]


# Hand-made segment layouts whose last round of output tiles is partly
# filled, so that, given a workspace, the grouped GEMM splits those tiles
# along K (one per tile configuration: large, medium, small and fp32).
SPLIT_CASES = {
    # name: (dtype, act, T, d, E, k, F, segment rows); the split runs only
    # where K >= 2048, so d (the up-projection's K) is at least that
    "large_relu": ("bf16", "relu", 1024, 2048, 4, 2, 2048, [700, 300, 512, 536]),
    "large_ragged": ("bf16", "relu", 1024, 2048, 4, 2, 2048, [1, 0, 1019, 1000]),
    # the SwiGLU epilogue on the large tile: gate and up columns paired, a
    # partly filled last column tile (F = 320 is 2.5 tiles of 128 outputs),
    # an odd slice count (d = 2112 is 33 slices of 64)
    "large_swiglu": ("bf16", "swiglu", 1024, 2048, 4, 2, 768, [700, 300, 512, 536]),
    "large_swiglu_ragged": ("bf16", "swiglu", 1024, 2112, 4, 2, 320, [1, 0, 1019, 1028]),
    # 256 mean rows with K >= 1024: the bf16 forward takes the large tile here
    "medium_swiglu": ("bf16", "swiglu", 512, 2048, 4, 2, 512, [300, 0, 257, 300]),
    # 128 mean rows per expert: the medium tile, whose waves hold one
    # 32-column block (16 gate and 16 up columns), with its SwiGLU tail store
    "medium_tile_swiglu": ("bf16", "swiglu", 512, 2048, 8, 2, 320, [200, 0, 130, 170, 128, 140, 120, 110]),
    # 64 mean rows per expert: the small tile, likewise one block per wave
    "small_swiglu": ("bf16", "swiglu", 512, 2048, 16, 2, 320, [64] * 14 + [1, 63]),
    "small_relu": ("bf16", "relu", 512, 2048, 16, 2, 512, [64] * 14 + [1, 63]),
    "f32_relu": ("f32", "relu", 512, 2048, 4, 1, 512, [130, 0, 200, 150]),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_expert_split_tail(name):
    dtype, act, T, d, E, k, F, seg = SPLIT_CASES[name]
    print(f"[ffn-split] {name}", flush=True)
    assert sum(seg) <= T * k and len(seg) == E
    p = moe.problem(T, d, E, k, F, act=act, dtype=dtype)
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    P = int(offsets[-1])
    rng = np.random.default_rng(4242 + len(name))
    n1 = 2 * F if act == "swiglu" else F
    x = moe_inputs._cast(rng.standard_normal((T, d)).astype(np.float32), dtype)
    src = rng.integers(0, T, size=P).astype(np.int32)
    xp = x[src]
    W1 = moe_inputs._cast((rng.standard_normal((E, n1, d)) / np.sqrt(d)).astype(np.float32), dtype)
    W2 = moe_inputs._cast((rng.standard_normal((E, d, F)) / np.sqrt(F)).astype(np.float32), dtype)
    hs = moe_inputs._cast(np.abs(rng.standard_normal((P, F))).astype(np.float32), dtype)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    rows_cap = T * k
    xp_d = torch.zeros(rows_cap, d, dtype=dt, device="cuda")
    xp_d[:P] = dev(xp)
    src_d = torch.full((rows_cap,), -1, dtype=torch.int32, device="cuda")
    src_d[:P] = dev(src)
    hs_d = torch.zeros(rows_cap, F, dtype=dt, device="cuda")
    hs_d[:P] = dev(hs)
    off_d, W1_d, W2_d = dev(offsets), dev(W1), dev(W2)
    # poisoned workspace: the split must write its partial tiles there
    ws = torch.full((moe.moe_workspace_size(p),), 0xFF, dtype=torch.uint8, device="cuda")
    h0 = torch.zeros(rows_cap, F, dtype=dt, device="cuda")
    h1, h2 = torch.zeros_like(h0), torch.zeros_like(h0)
    moe.moe_expert_up(p, xp_d, None, off_d, W1_d, h0)
    moe.moe_expert_up(p, xp_d, None, off_d, W1_d, h1, ws=ws)
    torch.cuda.synchronize()
    assert int((ws != 0xFF).sum()) > 0, "the K split did not run"
    moe.moe_expert_up(p, dev(x), src_d, off_d, W1_d, h2, ws=ws)
    y0 = torch.zeros(rows_cap, d, dtype=dt, device="cuda")
    y1 = torch.zeros_like(y0)
    moe.moe_expert_down(p, hs_d, off_d, W2_d, y0)
    moe.moe_expert_down(p, hs_d, off_d, W2_d, y1, ws=ws)
    torch.cuda.synchronize()
    act_c = oracle.SWIGLU if act == "swiglu" else oracle.RELU
    _y, ref_h = oracle.ffn_rows(xp, offsets, W1, W2, act_c, F, want_h=True)
    ref_y = oracle.down_rows(hs, offsets, W2)
    for got in (h0, h1, h2):
        assert maxrel(host(got)[:P], ref_h) <= TOL[dtype]
    assert np.array_equal(host(h1)[:P], host(h2)[:P])
    for got in (y0, y1):
        assert maxrel(host(got)[:P], ref_y) <= TOL[dtype]
    # rows past the kept ones are never written
    assert not host(h1)[P:].any() and not host(y1)[P:].any()


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("name", SMALL)
def test_combine(name):
    case = moe_inputs.get(name)
    inp = inputs(name, weights=False)
    print(f"[combine] {name}", flush=True)
    p = problem_of(case)
    _ze, _z32, idx, w, disp = oracle_route(case, inp)
    P = disp["P"]
    yp = moe_inputs._cast(RNG.standard_normal((max(P, 1), case.d)).astype(np.float32), case.dtype)
    w32 = w.astype(np.float32)
    y = torch.empty(case.T, case.d, dtype=torch_dtype(case), device="cuda")
    yp_d = torch.zeros(case.T * case.k, case.d, dtype=torch_dtype(case), device="cuda")
    yp_d[:P] = dev(yp[:P])
    moe.moe_combine(p, yp_d, dev(disp["slot"]), dev(w32), y)
    torch.cuda.synchronize()
    ref = oracle.combine(yp[:max(P, 1)], disp["slot"], w32.astype(np.float64), case.T)
    got = host(y)
    assert maxrel(got, ref) <= TOL[case.dtype]
    dropped_all = np.all(disp["slot"] < 0, axis=1)
    assert np.all(to_f64(got[dropped_all]) == 0.0)


# ------------------------------------------------------------------ whole layer
def check_forward(case, inp, out, tokens=None):
    _ze, z32, idx, w, disp = oracle_route(case, inp)
    assert np.array_equal(out["topk_idx"], idx)
    assert np.max(np.abs(out["topk_w"].astype(np.float64) - w)) <= TOPK_W_ATOL
    assert np.array_equal(out["counts"], disp["counts"])
    assert np.array_equal(out["offsets"], disp["offsets"])
    assert np.array_equal(out["slot"], disp["slot"])
    assert np.array_equal(out["src_token"][:disp["P"]], disp["src_token"])
    if case.logits == "gate":
        assert np.max(np.abs(out["logits"].astype(np.float64) - z32)) <= 1e-6 * max(1.0, np.max(np.abs(z32)))
    y_ref = oracle.forward_tokens(inp["x"], inp["W1"], inp["W2"], idx, w, disp["slot"], act_code(case), case.F,
                                  tokens)
    got = out["y"] if tokens is None else out["y"][tokens]
    err = maxrel(got, y_ref)
    assert err <= TOL[case.dtype], err
    dropped = np.all(disp["slot"] < 0, axis=1)
    if tokens is None:
        assert np.all(to_f64(out["y"][dropped]) == 0.0)
    return err, disp


@pytest.mark.parametrize("name", SMALL)
def test_forward_small(name):
    case = moe_inputs.get(name)
    inp = inputs(name)
    print(f"[forward] {name}", flush=True)
    out = run_forward(case, inp)
    err, disp = check_forward(case, inp, out)
    print(f"  max-abs-rel {err:.3e}, dropped {case.T * case.k - disp['P']}", flush=True)


def sample_tokens(case, inp, disp, n=24):
    """Random tokens, the first and last, hot and dropped ones; on the large
    tile (bf16, at least 512 rows per expert on average) also tokens whose
    rows reach every m-tile of every expert, and every row of the smallest
    tile that the last round of each expert GEMM splits along K."""
    T = case.T
    g = np.random.default_rng(case.seed)
    picks = {0, T - 1}
    picks.update(g.choice(T, size=min(n, T), replace=False).tolist())
    if "hot_tokens" in inp:
        picks.update(inp["hot_tokens"][:4].tolist())
    dropped_any = np.nonzero(np.any(disp["slot"] < 0, axis=1))[0]
    picks.update(dropped_any[:4].tolist())
    if uses_large_tile(case):
        G = torch.cuda.get_device_properties(0).multi_processor_count
        ntns = [(case.F + 127) // 128 if case.act == "swiglu" else (case.F + 255) // 256, (case.d + 255) // 256]
        picks.update(_tiles.covering_tokens(disp["offsets"], disp["src_token"], ntns, G).tolist())
    return np.array(sorted(picks), np.int32)


def uses_large_tile(case):
    rows = case.T * case.k // case.E
    C = oracle.capacity(case.T, case.E, case.k, case.cf)
    if C >= 0:
        rows = min(rows, C)
    return case.dtype == "bf16" and rows >= 512


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size_sampled(name):
    """Full sizes, same entry point and launch configuration as the benchmark:
    routing and permutation in full, outputs on sampled tokens."""
    case = moe_inputs.get(name)
    inp = inputs(name)
    print(f"[forward-full] {name}", flush=True)
    out = run_forward(case, inp)
    _ze, _z32, _idx, _w, disp = oracle_route(case, inp)
    toks = sample_tokens(case, inp, disp)
    err, _ = check_forward(case, inp, out, toks)
    print(f"  max-abs-rel {err:.3e} on {len(toks)} tokens, dropped {case.T * case.k - disp['P']}", flush=True)


def test_forward_large_t():
    """About a million tokens (given logits, capacity 1.0): routing and the
    permutation in full, outputs on sampled tokens."""
    case = moe_inputs.get("large_t_fwd")
    inp = inputs(case.name)
    print(f"[forward-large] {case.name} T={case.T}", flush=True)
    out = run_forward(case, inp)
    _ze, _z32, _idx, _w, disp = oracle_route(case, inp)
    toks = sample_tokens(case, inp, disp)
    err, _ = check_forward(case, inp, out, toks)
    print(f"  max-abs-rel {err:.3e} on {len(toks)} tokens, dropped {case.T * case.k - disp['P']}", flush=True)


def test_forward_deterministic_and_workspace_independent():
    case = moe_inputs.get("skywork_m_zipf_s")
    inp = inputs(case.name)
    a = run_forward(case, inp, ws_fill=0)
    b = run_forward(case, inp, ws_fill=0xFF)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("kind", ["T1", "E_equals_k", "k1", "single_expert", "heavy_drop", "all_to_one",
                                  "fp32_swiglu_norm", "cf_not_dyadic"])
def test_forward_edges(kind):
    print(f"[forward-edge] {kind}", flush=True)
    base = moe_inputs.get("mixtral_s").with_(bias="none")
    over = {}
    if kind == "T1":
        case = base.with_(name="edge_T1", T=1)
    elif kind == "E_equals_k":
        case = base.with_(name="edge_Ek", E=2, k=2, act="relu")
    elif kind == "k1":
        case = base.with_(name="edge_k1", k=1, normalize=True)
    elif kind == "single_expert":
        case = base.with_(name="edge_E1", E=1, k=1)
    elif kind == "heavy_drop":
        case = base.with_(name="edge_drop", cf=0.25, normalize=True)
    elif kind == "all_to_one":
        case = base.with_(name="edge_one", cf=0.5)
    elif kind == "cf_not_dyadic":
        # capacity from fp32(0.7): 0.7 * 600 * 2 / 8 = 105 in decimal, C = 105
        # from fp32(0.7) = 0.69999999; the Zipf bias of mixtral_s makes it bite
        case = moe_inputs.get("mixtral_s").with_(name="edge_cf07", cf=0.7)
        assert oracle.capacity(case.T, case.E, case.k, case.cf) == moe.moe_capacity(problem_of(case)) == 105
    else:
        case = base.with_(name="edge_f32", dtype="f32", x_std=0.5, normalize=True, lam=2.0, cf=1.0, T=300)
    # the Zipf-biased variant reuses mixtral_s's calibrated gate bias
    inp = moe_inputs.make(case, bias_override=moe_inputs.zipf_bias(moe_inputs.get("mixtral_s"))
                          if case.bias == "zipf" else None)
    if kind == "all_to_one":
        # every token's logits favour experts 5 then 2 (zero gate weight, fixed bias)
        inp["Wg"] = np.zeros_like(inp["Wg"])
        bg = np.zeros(case.E, np.float32)
        bg[5], bg[2] = 2.0, 1.0
        inp["bg"] = bg
    out = run_forward(case, inp)
    err, disp = check_forward(case, inp, out)
    print(f"  max-abs-rel {err:.3e}, dropped {case.T * case.k - disp['P']}", flush=True)
