"""Pins of the CPU oracle to things other than itself.

Each test ties one step of the oracle to a definition written out
independently (numpy / scipy library routines, brute force on tiny inputs,
closed forms, invariants the layer must satisfy).  A plausible slip in the
oracle -- a dropped term, a wrong sign or index, a transposed operand, a
swapped gate/up half, a sample instead of a population deviation, a wrong tie
or drop rule -- fails at least one of them.

Sources of the definitions: the MoE layer (gate picks k of n experts, weighted
mix) from the FastMoE announcement page, "§1 MoE 设计" and Fig. 1, and the
industry-overview page, "MoE的內涵"; Top-K routing from the Megatron-Core page,
"关键特性"; capacity and dropping from its "MoE负载均衡的挑战与应对" section;
the gating-logit normalisation from the Skywork-MoE news item, "技术创新 1", and
the Skywork slides, slide 6; SwiGLU's gate/up halves from the Megatron-Core
page, "权重转换要点"; ReLU experts from the FastMoE page, "特色三".
"""
import math

import numpy as np
import pytest
import scipy.special

import moe_inputs
import oracle

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- helpers
def dense_ffn(xf, W1e, W2e, act, F):
    """Textbook two-layer MLP in float64, written independently of the oracle."""
    if act == oracle.RELU:
        h = np.maximum(xf @ W1e.T, 0.0)
    else:
        g = xf @ W1e[:F].T
        u = xf @ W1e[F:].T
        h = g * scipy.special.expit(g) * u
    return h @ W2e.T


def brute_topk(z, k):
    """Selection and order from counting: expert e takes position
    #{e': z_e' > z_e} + #{e' < e: z_e' == z_e} when that is below k."""
    E = z.shape[0]
    pos = {}
    for e in range(E):
        r = sum(1 for f in range(E) if z[f] > z[e]) + sum(1 for f in range(e) if z[f] == z[e])
        if r < k:
            pos[r] = e
    return np.array([pos[j] for j in range(k)], np.int32)


def rand_bf16(shape, std=1.0):
    return moe_inputs.f32_to_bf16_bits(RNG.standard_normal(shape).astype(np.float32) * np.float32(std))


# ---------------------------------------------------------------- bf16 widening
def test_bf16_widening_exact():
    assert oracle.bf16_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert oracle.bf16_to_f64(np.array([0xC000], np.uint16))[0] == -2.0
    assert oracle.bf16_to_f64(np.array([0x3FC0], np.uint16))[0] == 1.5
    assert oracle.bf16_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -133  # smallest subnormal
    assert oracle._load().orc_bf16_to_double(0x4049) == 3.140625
    # the generator's RNE rounding: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert moe_inputs.f32_to_bf16_bits(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80
    assert moe_inputs.f32_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82


# ---------------------------------------------------------------- gate logits
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_logits_match_library_matmul(dtype):
    T, d, E = 37, 96, 5
    x = RNG.standard_normal((T, d)).astype(np.float32)
    W = RNG.standard_normal((E, d)).astype(np.float32) * np.float32(0.1)
    bg = RNG.standard_normal(E).astype(np.float32)
    if dtype == "bf16":
        x, W = moe_inputs.f32_to_bf16_bits(x), moe_inputs.f32_to_bf16_bits(W)
    ze, z32 = oracle.gate_logits(x, W, bg)
    ref = oracle.to_f64(x) @ oracle.to_f64(W).T + bg.astype(np.float64)[None, :]
    assert np.max(np.abs(ze - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    assert np.array_equal(z32, ref.astype(np.float32)) or np.max(np.abs(z32 - ref)) <= 2 ** -23 * np.max(np.abs(ref))
    # without a bias the bias term must vanish
    ze0, _ = oracle.gate_logits(x, W, None)
    assert np.allclose(ze0 + bg[None, :], ze, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- top-k selection
@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (3, 2), (4, 2), (5, 3), (6, 6), (6, 2)])
def test_topk_brute_force_with_ties(E, k):
    for trial in range(200):
        # few distinct values -> many ties; include signed zeros
        z = RNG.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0], np.float32), size=E)
        got = oracle.topk(z, k)
        assert np.array_equal(got, brute_topk(z, k)), (z, got)
        # library cross-check: stable sort by descending key, ties by index
        lib = sorted(range(E), key=lambda e: (-float(z[e]), e))[:k]
        assert got.tolist() == lib


def test_topk_signed_zero_and_ties_go_to_lower_index():
    z = np.array([-0.0, 0.0, -0.0, 0.0], np.float32)
    assert oracle.topk(z, 2).tolist() == [0, 1]
    z = np.array([0.0, -0.0, 1.0, -1.0], np.float32)
    assert oracle.topk(z, 3).tolist() == [2, 0, 1]


def test_route_selection_invariant_to_normalisation_and_exact_scaling():
    T, E, k = 64, 16, 3
    z = RNG.standard_normal((T, E)).astype(np.float32)
    idx0, _ = oracle.route(z, k)
    for norm, lam in [(True, 1.0), (True, 0.25), (True, 7.0)]:
        idx1, _ = oracle.route(z, k, norm, lam)
        assert np.array_equal(idx0, idx1)
    idx2, _ = oracle.route(z * np.float32(4.0), k)  # exact in fp32
    assert np.array_equal(idx0, idx2)


# ---------------------------------------------------------------- normalisation
def test_normalisation_zero_mean_unit_variance():
    for E in (2, 8, 16, 512):
        for lam in (1.0, 0.5, 3.0):
            z = (RNG.standard_normal(E) * 3 + 1.7).astype(np.float32)
            zt = oracle.normalize(z, lam)
            s = zt / lam
            assert abs(s.mean()) < 1e-12
            assert abs((s * s).mean() - 1.0) < 1e-12
            # library form: population standard deviation (numpy's default ddof=0)
            zd = z.astype(np.float64)
            ref = lam * (zd - zd.mean()) / zd.std()
            assert np.max(np.abs(zt - ref)) < 1e-12


def test_normalisation_constant_logits_give_uniform_probs():
    z = np.full(8, 0.75, np.float32)
    assert np.all(oracle.normalize(z, 1.0) == 0.0)
    p = oracle.gate_probs(z, True, 1.0)
    assert np.allclose(p, 1.0 / 8, rtol=0, atol=1e-15)


def test_normalisation_sharpens_with_lambda():
    # d log p_max / d lambda = zt_max/lambda - E_p[zt/lambda] >= 0: the top
    # probability can only grow with lambda ("sharper" router probabilities).
    for _ in range(50):
        z = RNG.standard_normal(16).astype(np.float32)
        prev = 0.0
        for lam in (0.1, 0.3, 0.5, 1.0, 1.5, 2.0, 4.0, 8.0):
            pm = oracle.gate_probs(z, True, lam).max()
            assert pm >= prev - 1e-15
            prev = pm


# ---------------------------------------------------------------- softmax
def test_softmax_library_and_closed_forms():
    for E in (1, 2, 7, 64):
        s = RNG.standard_normal(E) * 4
        p = oracle.softmax(s)
        assert abs(p.sum() - 1.0) < 1e-14
        assert np.max(np.abs(p - scipy.special.softmax(s))) < 1e-15
        assert np.max(np.abs(oracle.softmax(s + 123.0) - p)) < 1e-14  # shift invariance
    assert oracle.softmax(np.array([5.0]))[0] == 1.0
    p = oracle.softmax(np.array([1.0, 0.0]))
    assert abs(p[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


def test_unnormalised_probs_are_softmax_of_fp32_logits():
    z = RNG.standard_normal(10).astype(np.float32)
    p = oracle.gate_probs(z, False, 1.0)
    assert np.max(np.abs(p - scipy.special.softmax(z.astype(np.float64)))) < 1e-15


# ---------------------------------------------------------------- weights
def test_topk_weights_are_softmax_entries():
    T, E, k = 50, 12, 4
    z = RNG.standard_normal((T, E)).astype(np.float32)
    for norm in (False, True):
        idx, w, p = oracle.route(z, k, norm, 1.0, want_p=True)
        assert np.array_equal(w, np.take_along_axis(p, idx.astype(np.int64), axis=1))
        assert np.all(w.sum(axis=1) <= 1.0 + 1e-15)
        # selection order = descending weight (softmax is increasing)
        assert np.all(np.diff(w, axis=1) <= 1e-15)
    idx, w = oracle.route(z, E)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-14


# ---------------------------------------------------------------- capacity / dispatch
def test_capacity_formula():
    assert oracle.capacity(4096, 16, 2, 1.25) == 640
    assert oracle.capacity(10, 3, 1, 1.0) == 4          # ceil(10/3)
    assert oracle.capacity(10, 3, 1, 0.0) == -1
    assert oracle.capacity(10, 3, 1, -2.0) == -1
    assert oracle.capacity(8, 4, 2, 1e-30) == 1
    assert oracle.capacity(4096, 8, 2, 0.25) == 256


# The capacity factor is a single-precision number; C is the exact ceiling of
# fp32(cf) * T * k / E, checked here with rational arithmetic (no floating
# point).  Factors that are not dyadic (0.1, 0.3, 0.7, 1.1, 1/3) land just
# above or below an integer, where a product or quotient rounded the wrong
# way would move C by one.
@pytest.mark.parametrize("T,E,k,cf", [(100, 1, 1, 0.3), (1000, 10, 1, 0.3), (10, 1, 1, 0.3), (100, 1, 1, 0.1),
                                      (100, 1, 1, 0.7), (100, 1, 1, 1.1), (1000, 4, 2, 0.3), (300, 3, 2, 1 / 3),
                                      (4096, 16, 2, 1.25), (16384, 512, 2, 0.25), (1 << 24, 1024, 8, 0.7),
                                      (777, 40, 8, 1.0), (5, 7, 3, 2.2)])
def test_capacity_is_exact_ceiling_of_fp32_factor(T, E, k, cf):
    from fractions import Fraction
    exact = Fraction(float(np.float32(cf))) * T * k / E
    assert oracle.capacity(T, E, k, cf) == math.ceil(exact)


def brute_dispatch(idx, E, C):
    T, k = idx.shape
    slot = np.full((T, k), -1, np.int64)
    counts = np.array([(idx == e).sum() for e in range(E)])
    kept = counts if C < 0 else np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept)])
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            r = sum(1 for t2 in range(t) for j2 in range(k) if idx[t2, j2] == e)
            if C < 0 or r < C:
                slot[t, j] = offsets[e] + r
    return counts, offsets, slot


@pytest.mark.parametrize("T,E,k,cf", [(1, 1, 1, 0.0), (9, 3, 2, 0.0), (40, 5, 2, 0.5), (33, 4, 4, 1.0),
                                      (60, 6, 1, 0.25), (20, 8, 3, 100.0)])
def test_dispatch_brute_force(T, E, k, cf):
    z = RNG.standard_normal((T, E)).astype(np.float32)
    z[:, 0] += 1.0  # skew towards expert 0 so capacity bites
    idx, _ = oracle.route(z, k)
    C = oracle.capacity(T, E, k, cf)
    got = oracle.dispatch(idx, E, C)
    counts, offsets, slot = brute_dispatch(idx, E, C)
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["slot"], slot)
    assert got["counts"].sum() == T * k
    dropped = T * k - got["offsets"][E]
    assert dropped == int((got["slot"] < 0).sum())
    if C < 0:
        assert dropped == 0
    P = got["P"]
    st = got["src_token"]
    for t in range(T):
        for j in range(k):
            if got["slot"][t, j] >= 0:
                assert st[got["slot"][t, j]] == t


def test_dispatch_matches_library_stable_sort():
    T, E, k = 300, 7, 3
    idx, _ = oracle.route(RNG.standard_normal((T, E)).astype(np.float32), k)
    got = oracle.dispatch(idx, E, -1)
    order = np.argsort(idx.ravel(), kind="stable")   # token-major list, stable by expert
    assert np.array_equal(got["src_token"], (order // k).astype(np.int32))
    # huge capacity is the same as dropless
    big = oracle.dispatch(idx, E, 10 ** 9)
    for key in ("counts", "offsets", "slot", "src_token"):
        assert np.array_equal(big[key], got[key])


def test_drops_keep_earliest_tokens():
    T, E, k = 30, 3, 1
    idx = np.zeros((T, k), np.int32)          # every token on expert 0
    got = oracle.dispatch(idx, E, 4)
    assert got["slot"][:4, 0].tolist() == [0, 1, 2, 3]
    assert np.all(got["slot"][4:, 0] == -1)
    assert got["offsets"].tolist() == [0, 4, 4, 4]


# ---------------------------------------------------------------- expert FFN and layer
@pytest.mark.parametrize("act", [oracle.RELU, oracle.SWIGLU])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_is_dense_ffn(act, dtype):
    # E = 1, k = 1: the only expert has probability 1 and the layer is a dense FFN.
    T, d, F = 23, 64, 128
    n1 = 2 * F if act == oracle.SWIGLU else F
    x = RNG.standard_normal((T, d)).astype(np.float32)
    Wg = RNG.standard_normal((1, d)).astype(np.float32)
    W1 = (RNG.standard_normal((1, n1, d)) * 0.1).astype(np.float32)
    W2 = (RNG.standard_normal((1, d, F)) * 0.1).astype(np.float32)
    if dtype == "bf16":
        x, Wg, W1, W2 = (moe_inputs.f32_to_bf16_bits(a) for a in (x, Wg, W1, W2))
    out = oracle.moe_forward(x, Wg, None, W1, W2, k=1, F=F, act=act)
    ref = dense_ffn(oracle.to_f64(x), oracle.to_f64(W1)[0], oracle.to_f64(W2)[0], act, F)
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("act", [oracle.RELU, oracle.SWIGLU])
def test_identical_experts_scale_by_weight_sum(act):
    T, d, E, k, F = 31, 64, 6, 3, 64
    n1 = 2 * F if act == oracle.SWIGLU else F
    x = rand_bf16((T, d))
    Wg = rand_bf16((E, d), 0.3)
    W1_one = rand_bf16((1, n1, d), 0.1)
    W2_one = rand_bf16((1, d, F), 0.1)
    W1 = np.repeat(W1_one, E, axis=0)
    W2 = np.repeat(W2_one, E, axis=0)
    out = oracle.moe_forward(x, Wg, None, W1, W2, k=k, F=F, act=act)
    ref = dense_ffn(oracle.to_f64(x), oracle.to_f64(W1_one)[0], oracle.to_f64(W2_one)[0], act, F)
    ref = ref * out["topk_w"].sum(axis=1)[:, None]
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("act", [oracle.RELU, oracle.SWIGLU])
@pytest.mark.parametrize("norm,cf", [(False, 0.0), (True, 0.0), (False, 0.6), (True, 1.0)])
def test_layer_equals_dense_mixture_formulation(act, norm, cf):
    """Shazeer-style dense form: y_t = sum_e g_te FFN_e(x_t) with g_te = p_te when
    expert e is a kept choice of token t, else 0 -- computed over every expert
    by a second, vectorised code path."""
    T, d, E, k, F = 16, 64, 6, 2, 64
    n1 = 2 * F if act == oracle.SWIGLU else F
    x = rand_bf16((T, d))
    Wg = rand_bf16((E, d), 0.3)
    bg = (RNG.standard_normal(E) * 0.5).astype(np.float32)
    W1 = rand_bf16((E, n1, d), 0.1)
    W2 = rand_bf16((E, d, F), 0.1)
    lam = 1.0
    out = oracle.moe_forward(x, Wg, bg, W1, W2, k=k, F=F, act=act, normalize_flag=norm, lam=lam, cf=cf)
    xf = oracle.to_f64(x)
    # independent gate: logits in float64, rounded to fp32 for the selection key
    z = (xf @ oracle.to_f64(Wg).T + bg.astype(np.float64)).astype(np.float32)
    zd = z.astype(np.float64)
    s = lam * (zd - zd.mean(1, keepdims=True)) / zd.std(1, keepdims=True) if norm else zd
    p = scipy.special.softmax(s, axis=1)
    order = np.array([sorted(range(E), key=lambda e: (-float(z[t, e]), e))[:k] for t in range(T)])
    C = math.ceil(cf * T * k / E) if cf > 0 else None
    g = np.zeros((T, E))
    seen = np.zeros(E, int)
    for t in range(T):
        for j in range(k):
            e = order[t, j]
            if C is None or seen[e] < C:
                g[t, e] = p[t, e]
            seen[e] += 1
    ref = np.zeros((T, d))
    for e in range(E):
        ref += g[:, e:e + 1] * dense_ffn(xf, oracle.to_f64(W1)[e], oracle.to_f64(W2)[e], act, F)
    assert np.array_equal(out["topk_idx"], order.astype(np.int32))
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.max(np.abs(ref))
    if cf > 0:
        dropped = (out["slot"] < 0).sum()
        assert out["counts"].sum() - out["offsets"][-1] == dropped


def test_fully_dropped_token_outputs_zero():
    T, d, E, k, F = 8, 64, 2, 1, 64
    x = rand_bf16((T, d))
    Wg = np.zeros((E, d), np.uint16)           # all logits 0 -> every token picks expert 0
    W1 = rand_bf16((E, F, d), 0.1)
    W2 = rand_bf16((E, d, F), 0.1)
    out = oracle.moe_forward(x, Wg, None, W1, W2, k=k, F=F, act=oracle.RELU, cf=0.5)   # C = 2
    assert out["C"] == 2
    assert np.all(out["topk_idx"] == 0)
    assert np.all(out["y"][2:] == 0.0)
    assert np.any(out["y"][:2] != 0.0)


def test_ffn_rows_and_combine_recompose_forward():
    T, d, E, k, F = 40, 64, 5, 2, 128
    x = rand_bf16((T, d))
    Wg = rand_bf16((E, d), 0.3)
    W1 = rand_bf16((E, 2 * F, d), 0.1)
    W2 = rand_bf16((E, d, F), 0.1)
    out = oracle.moe_forward(x, Wg, None, W1, W2, k=k, F=F, act=oracle.SWIGLU, cf=0.7)
    xp = x[out["src_token"]]
    yp = oracle.ffn_rows(xp, out["offsets"], W1, W2, oracle.SWIGLU, F)
    # expert of each row from offsets: compare to a direct per-row call
    for r in (0, out["P"] - 1) + tuple(out["offsets"][1:-1]):
        if r >= out["P"]:
            continue
        e = int(np.searchsorted(out["offsets"], r, side="right") - 1)
        ref = oracle.expert_ffn(W1, W2, e, oracle.to_f64(xp[r]), oracle.SWIGLU, F)
        assert np.array_equal(yp[r], ref)
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            s = out["slot"][t, j]
            if s >= 0:
                y[t] += out["topk_w"][t, j] * yp[s]
    assert np.max(np.abs(y - out["y"])) <= 1e-12 * np.max(np.abs(y))
    # the oracle's combine on float64-exact expert outputs
    yp32 = yp.astype(np.float32)
    yc = oracle.combine(yp32, out["slot"], out["topk_w"], T)
    yref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            s = out["slot"][t, j]
            if s >= 0:
                yref[t] += out["topk_w"][t, j] * yp32[s].astype(np.float64)
    assert np.max(np.abs(yc - yref)) <= 1e-13 * np.max(np.abs(yref))


def test_forward_token_subset_matches_full():
    T, d, E, k, F = 24, 64, 4, 2, 64
    x = rand_bf16((T, d))
    Wg = rand_bf16((E, d), 0.3)
    W1 = rand_bf16((E, F, d), 0.1)
    W2 = rand_bf16((E, d, F), 0.1)
    full = oracle.moe_forward(x, Wg, None, W1, W2, k=k, F=F, act=oracle.RELU)
    toks = np.array([3, 17, 0, 23], np.int32)
    sub = oracle.forward_tokens(x, W1, W2, full["topk_idx"], full["topk_w"], full["slot"], oracle.RELU, F, toks)
    assert np.array_equal(sub, full["y"][toks])


# ---------------------------------------------------------------- calibrated inputs
@pytest.mark.parametrize("name", [n for n, c in moe_inputs.CASES.items() if c.bias == "zipf"])
def test_zipf_bias_realises_target_shares(name):
    case = moe_inputs.get(name)
    inp = moe_inputs.make(case, weights=False)
    _ze, z32 = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
    idx, _ = oracle.route(z32, case.k)
    f = np.bincount(idx.ravel(), minlength=case.E) / (case.T * case.k)
    q = moe_inputs.zipf_shares(case.E, case.zipf_s)
    assert np.max(np.abs(f - q)) < 0.005, (f, q)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_down_rows_is_second_linear_layer(dtype):
    E, d, F = 4, 64, 128
    offsets = np.array([0, 5, 5, 12, 20], np.int32)   # expert 1 empty
    h = RNG.standard_normal((20, F)).astype(np.float32)
    W2 = (RNG.standard_normal((E, d, F)) * 0.1).astype(np.float32)
    if dtype == "bf16":
        h, W2 = moe_inputs.f32_to_bf16_bits(h), moe_inputs.f32_to_bf16_bits(W2)
    out = oracle.down_rows(h, offsets, W2)
    h64, W64 = oracle.to_f64(h), oracle.to_f64(W2)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        ref = h64[a:b] @ W64[e].T
        assert np.max(np.abs(out[a:b] - ref), initial=0.0) <= 1e-12 * max(1.0, np.max(np.abs(ref), initial=0.0))
    # consistent with the whole FFN: down(h of ffn_rows) == ffn_rows
    xp = moe_inputs.f32_to_bf16_bits(RNG.standard_normal((20, d)).astype(np.float32))
    W1 = moe_inputs.f32_to_bf16_bits((RNG.standard_normal((E, F, d)) * 0.1).astype(np.float32))
    W2b = moe_inputs.f32_to_bf16_bits(W2) if dtype == "f32" else W2
    full, hh = oracle.ffn_rows(xp, offsets, W1, W2b, oracle.RELU, F, want_h=True)
    assert hh.shape == (20, F)
    ref = np.stack([hh[r] @ oracle.to_f64(W2b)[int(np.searchsorted(offsets, r, side="right") - 1)].T
                    for r in range(20)])
    assert np.max(np.abs(full - ref)) <= 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------------- router by-products
# Definitions read for the pages' unnamed formulas (Megatron-Core page, "MoE负载
# 均衡的挑战与应对" and "关键特性": auxiliary balancing loss, Z-Loss; Skywork
# news item, "技术创新 2", and slides, slide 7: drop-rate-driven coefficient):
# f_e = counts/(T k), P_e = mean_t p[t,e], aux = E sum f P, z = mean (lse z)^2,
# drop = dropped/(T k).

def test_router_stats_uniform_and_balanced_closed_forms():
    T, E, k = 37, 6, 2
    # all logits equal: P_e = 1/E, so aux = sum_e f_e = 1 whatever the counts;
    # logsumexp = c + log E
    z = np.full((T, E), 0.75, np.float32)
    counts = np.array([20, 0, 30, 4, 10, 10], np.int32)
    st = oracle.router_stats(z, counts, T * k, k)
    assert np.allclose(st["mean_prob"], 1.0 / E, rtol=0, atol=1e-15)
    assert abs(st["aux"] - 1.0) < 1e-14
    assert abs(st["z_loss"] - (0.75 + math.log(E)) ** 2) < 1e-12
    assert st["drop_rate"] == 0.0
    # perfectly balanced counts: f_e = 1/E, so aux = sum_e P_e = 1 for any logits
    T = 36
    z = RNG.standard_normal((T, E)).astype(np.float32) * 3
    bal = oracle.router_stats(z, np.full(E, T * k // E, np.int32), T * k, k)
    assert abs(bal["aux"] - 1.0) < 1e-13


def test_router_stats_against_library_routines():
    T, E, k = 53, 7, 3
    z = (RNG.standard_normal((T, E)) * 2).astype(np.float32)
    idx, _w = oracle.route(z, k)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    st = oracle.router_stats(z, counts, T * k - 5, k)
    p = scipy.special.softmax(z.astype(np.float64), axis=1)
    lse = scipy.special.logsumexp(z.astype(np.float64), axis=1)
    assert np.allclose(st["mean_prob"], p.mean(axis=0), rtol=1e-13, atol=0)
    assert np.allclose(st["frac"], counts / (T * k), rtol=0, atol=1e-16)
    assert abs(st["aux"] - E * np.dot(counts / (T * k), p.mean(axis=0))) < 1e-13
    assert abs(st["z_loss"] - np.mean(lse ** 2)) < 1e-12 * max(1.0, np.mean(lse ** 2))
    assert abs(st["drop_rate"] - 5 / (T * k)) < 1e-16
    # invariants: both distributions sum to one
    assert abs(st["mean_prob"].sum() - 1.0) < 1e-13 and abs(st["frac"].sum() - 1.0) < 1e-15


def test_router_stats_normalised_probs_are_affine_invariant():
    # standardisation removes any positive scale and shift of a token's logits,
    # so the normalised mean probabilities do not move; the Z-loss (raw
    # logits) shifts by the closed form lse(z + c) = lse(z) + c
    T, E, k = 40, 9, 2
    z = RNG.standard_normal((T, E)).astype(np.float32)
    counts = np.full(E, 1, np.int32)
    a = oracle.router_stats(z, counts, T * k, k, True, 1.0)
    z2 = (z * np.float32(4.0) + np.float32(2.0)).astype(np.float32)
    b = oracle.router_stats(z2, counts, T * k, k, True, 1.0)
    assert np.allclose(a["mean_prob"], b["mean_prob"], rtol=1e-6)
    c = 3.0
    zs = (z.astype(np.float64) + c).astype(np.float32)
    lse = scipy.special.logsumexp(zs.astype(np.float64), axis=1)
    assert abs(oracle.router_stats(zs, counts, T * k, k)["z_loss"] - np.mean(lse ** 2)) < 1e-12 * np.mean(lse ** 2)
    # lambda sharpens: the top expert's mean probability grows with lambda
    lo = oracle.router_stats(z, counts, T * k, k, True, 0.5)["mean_prob"]
    hi = oracle.router_stats(z, counts, T * k, k, True, 2.0)["mean_prob"]
    p_lo = np.array([oracle.gate_probs(z[t], True, 0.5) for t in range(T)])
    assert np.allclose(lo, p_lo.mean(axis=0), rtol=1e-13)
    assert abs(hi.sum() - 1) < 1e-13 and not np.allclose(lo, hi)


def test_router_stats_drop_rate_matches_dispatch():
    T, E, k = 300, 8, 2
    z = (RNG.standard_normal((T, E)) + np.linspace(2, 0, E)).astype(np.float32)
    idx, _ = oracle.route(z, k)
    C = oracle.capacity(T, E, k, 0.5)
    disp = oracle.dispatch(idx, E, C)
    st = oracle.router_stats(z, disp["counts"], disp["P"], k)
    dropped = int((disp["slot"] < 0).sum())
    assert dropped > 0 and abs(st["drop_rate"] - dropped / (T * k)) < 1e-16
    # f is measured before the clip: a hot expert's share exceeds C / (T k)
    assert st["frac"].max() > C / (T * k)


# ---------------------------------------------------------------- shared expert
# DeepSeekMoE-style shared expert (industry overview page, "MoE未來重點研究方向"
# item 4): an expert every token goes through, added with weight one.

@pytest.mark.parametrize("act", [oracle.RELU, oracle.SWIGLU])
def test_shared_expert_identity_weights_closed_form(act):
    T, d = 23, 64
    x = RNG.standard_normal((T, d)).astype(np.float32)
    eye = np.eye(d, dtype=np.float32)
    Ws1 = eye if act == oracle.RELU else np.concatenate([eye, eye])
    ys = oracle.shared_expert(x, Ws1, eye, act, d)
    xf = x.astype(np.float64)
    ref = np.maximum(xf, 0) if act == oracle.RELU else xf * scipy.special.expit(xf) * xf
    assert np.allclose(ys, ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("act", [oracle.RELU, oracle.SWIGLU])
def test_shared_expert_is_dense_ffn_and_adds_unweighted(act):
    T, d, F, E, k = 31, 64, 128, 5, 2
    n1 = 2 * F if act == oracle.SWIGLU else F
    x = moe_inputs.f32_to_bf16_bits(RNG.standard_normal((T, d)).astype(np.float32))
    Ws1 = moe_inputs.f32_to_bf16_bits((RNG.standard_normal((n1, d)) * 0.1).astype(np.float32))
    Ws2 = moe_inputs.f32_to_bf16_bits((RNG.standard_normal((d, F)) * 0.1).astype(np.float32))
    ys = oracle.shared_expert(x, Ws1, Ws2, act, F)
    ref = dense_ffn(oracle.to_f64(x), oracle.to_f64(Ws1), oracle.to_f64(Ws2), act, F)
    assert np.allclose(ys, ref, rtol=1e-12, atol=1e-12)
    # the combine adds it with weight one on top of the routed mix
    W1 = moe_inputs.f32_to_bf16_bits((RNG.standard_normal((E, n1, d)) * 0.1).astype(np.float32))
    W2 = moe_inputs.f32_to_bf16_bits((RNG.standard_normal((E, d, F)) * 0.1).astype(np.float32))
    z = RNG.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route(z, k)
    disp = oracle.dispatch(idx, E, oracle.capacity(T, E, k, 0.7))
    yp = oracle.ffn_rows(x[disp["src_token"]], disp["offsets"], W1, W2, act, F).astype(np.float32)
    routed = oracle.combine(yp, disp["slot"], w, T)
    both = oracle.combine_shared(yp, disp["slot"], w, ys)
    assert np.array_equal(both, ys + routed)
    # a token whose choices were all dropped still gets the shared expert
    gone = np.all(disp["slot"] < 0, axis=1)
    if gone.any():
        assert np.array_equal(both[gone], ys[gone])
    # zero shared weights leave the routed layer
    zero = oracle.shared_expert(x, Ws1, np.zeros_like(Ws2), act, F)
    assert not zero.any()


# ---------------------------------------------------------------- FP8 experts
# OCP FP8 E4M3 codes with power-of-two row scales (Skywork-MoE FP8 checkpoint and
# "4090推理" FP8 inference; Megatron-Core page "关键特性": FP8 among the coming
# features).  torch's float8_e4m3fn is the independent reference for the format.
import torch  # noqa: E402


def torch_e4m3(v):
    """Codes of in-range values by torch's own conversion (ties to even)."""
    t = torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_and_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    finite = ~np.isnan(ref)
    assert finite.sum() == 254 and np.array_equal(ours[finite], ref[finite]) and np.isnan(ours[~finite]).all()
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    # every finite code is its own nearest code
    assert np.array_equal(oracle.e4m3_encode(ours[finite]), codes[finite])


def test_e4m3_encode_nearest_even_and_saturating():
    v = np.concatenate([RNG.uniform(-448, 448, 3000), RNG.standard_normal(3000) * 0.01,
                        RNG.uniform(-2 ** -6, 2 ** -6, 1000)]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(v), torch_e4m3(v))
    # exact midpoints between neighbouring codes go to the even mantissa
    vals = oracle.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    enc = oracle.e4m3_encode(mids)
    assert np.all(enc % 2 == 0)
    assert np.array_equal(enc, torch_e4m3(mids))
    # saturation instead of NaN above the largest finite value
    assert list(oracle.e4m3_encode([448.0, 449.0, 464.0, 470.0, 479.9, 480.0, 1e6, -1e6, -470.0])) == \
        [0x7E] * 7 + [0xFE, 0xFE]


def test_fp8_row_scale_is_smallest_power_of_two():
    for amax in list(RNG.uniform(1e-6, 1e4, 500)) + [448.0, 224.0, 224.0001, 1.0, 0.875 * 2 ** -3]:
        e = oracle.fp8_scale_exp(amax)
        assert amax <= 448 * 2.0 ** e and amax > 448 * 2.0 ** (e - 1)
    assert oracle.fp8_scale_exp(0.0) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_fp8_quant_rows_against_independent_quantiser(dtype):
    R, K = 37, 96
    v = (RNG.standard_normal((R, K)) * np.exp(RNG.uniform(-8, 8, (R, 1)))).astype(np.float32)
    v[3] = 0.0
    src = v if dtype == "f32" else moe_inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v.astype(np.float64)
    vals = oracle.to_f64(src) if dtype != "f64" else src
    codes, scales = oracle.quant_rows_fp8(src)
    for r in range(R):
        amax = np.abs(vals[r]).max()
        m, x = np.frexp(amax)
        e = 0 if amax == 0 else (x - 9 if m <= 0.875 else x - 8)
        assert scales[r] == np.float32(2.0 ** e)
        assert np.array_equal(codes[r], torch_e4m3(vals[r] / 2.0 ** e))
    deq = oracle.e4m3_decode(codes) * scales[:, None]
    # within half a code step: relative 2^-4 for normals
    assert np.all(np.abs(deq - vals) <= np.abs(vals) * 2.0 ** -4 + scales[:, None] * 2.0 ** -10)
    assert not codes[3].any() and scales[3] == 1.0


@pytest.mark.parametrize("act", [oracle.RELU, oracle.SWIGLU])
def test_fp8_ffn_is_dequantised_dense_ffn(act):
    E, d, F, n = 3, 64, 128, 41
    n1 = 2 * F if act == oracle.SWIGLU else F
    W1 = moe_inputs.f32_to_bf16_bits((RNG.standard_normal((E, n1, d)) * 0.05).astype(np.float32))
    W2 = moe_inputs.f32_to_bf16_bits((RNG.standard_normal((E, d, F)) * 0.05).astype(np.float32))
    W1q, w1s = oracle.quant_weights_fp8(W1)
    W2q, w2s = oracle.quant_weights_fp8(W2)
    x = moe_inputs.f32_to_bf16_bits(RNG.standard_normal((n, d)).astype(np.float32))
    xq, xs = oracle.quant_rows_fp8(x)
    offsets = np.array([0, 15, 15, n], np.int32)
    out, h = oracle.ffn_rows_fp8(xq, xs, offsets, W1q, w1s, W2q, w2s, act, F, want_h=True)
    W1d = oracle.e4m3_decode(W1q) * w1s[:, :, None]
    W2d = oracle.e4m3_decode(W2q) * w2s[:, :, None]
    xd = oracle.e4m3_decode(xq) * xs[:, None]
    for r in range(n):
        e = 0 if r < 15 else 2
        u = W1d[e] @ xd[r]
        hr = np.maximum(u, 0) if act == oracle.RELU else u[:F] * scipy.special.expit(u[:F]) * u[F:]
        assert np.allclose(h[r], hr, rtol=1e-12, atol=1e-14)
        # h is quantised per row by the independent quantiser before the down layer
        m, xe = np.frexp(np.abs(hr).max())
        es = xe - 9 if m <= 0.875 else xe - 8
        hd = torch.from_numpy((hr / 2.0 ** es).astype(np.float32)).to(torch.float8_e4m3fn).double().numpy() * 2.0 ** es
        assert np.allclose(out[r], W2d[e] @ hd, rtol=1e-12, atol=1e-14)
    # the down layer alone on given quantised rows
    hq, hs = oracle.quant_rows_fp8(h)
    down = oracle.down_rows_fp8(hq, hs, offsets, W2q, w2s)
    assert np.allclose(down, out, rtol=1e-12, atol=1e-14)


def test_fp8_forward_tokens_recomposes_rows_and_combine():
    T, d, E, k, F = 60, 64, 4, 2, 64
    x = moe_inputs.f32_to_bf16_bits(RNG.standard_normal((T, d)).astype(np.float32))
    W1q, w1s = oracle.quant_weights_fp8(moe_inputs.f32_to_bf16_bits(
        (RNG.standard_normal((E, 2 * F, d)) * 0.05).astype(np.float32)))
    W2q, w2s = oracle.quant_weights_fp8(moe_inputs.f32_to_bf16_bits(
        (RNG.standard_normal((E, d, F)) * 0.05).astype(np.float32)))
    z = RNG.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route(z, k)
    disp = oracle.dispatch(idx, E, oracle.capacity(T, E, k, 0.8))
    y = oracle.forward_tokens_fp8(x, W1q, w1s, W2q, w2s, idx, w, disp["slot"], oracle.SWIGLU, F)
    xq, xs = oracle.quant_rows_fp8(x)
    src = disp["src_token"]
    yp = oracle.ffn_rows_fp8(xq[src], xs[src], disp["offsets"], W1q, w1s, W2q, w2s, oracle.SWIGLU, F)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if disp["slot"][t, j] >= 0:
                ref[t] += w[t, j] * yp[disp["slot"][t, j]]
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-15)
    assert not y[np.all(disp["slot"] < 0, axis=1)].any()


# ---------------------------------------------------------------- backward
# The layer's gradient (training is what the pages measure: Skywork news "训练
# Infra", FastMoE page "特色三", Megatron-Core page "训练效果与性能实测").  Pinned
# against torch autograd in float64 on an independent forward written here, and
# against central differences of the forward oracle.

def torch_layer_grads(x, Wg, bg, W1, W2, z32, idx, slot, dy, act, F, normalize, lam):
    """Independent float64 forward with autograd.  The logits take the fp32
    values the routing used (straight-through: value z32, gradient of z)."""
    f64 = lambda a: torch.tensor(oracle.to_f64(np.asarray(a)), dtype=torch.float64, requires_grad=True)
    xt, W1t, W2t = f64(x), f64(W1), f64(W2)
    Wgt = f64(Wg) if Wg is not None else None
    bgt = torch.tensor(np.asarray(bg, np.float64), requires_grad=True) if bg is not None else None
    zv = torch.tensor(np.asarray(z32, np.float64))
    if Wgt is not None:
        z = xt @ Wgt.T + (bgt if bgt is not None else 0.0)
        z = z + (zv - z).detach()
    else:
        z = zv
    if normalize:
        mu = z.mean(dim=1, keepdim=True)
        sd = ((z - mu) ** 2).mean(dim=1, keepdim=True).sqrt()
        s = torch.where(sd > 0, lam * (z - mu) / torch.where(sd > 0, sd, torch.ones_like(sd)), torch.zeros_like(z))
    else:
        s = z
    p = torch.softmax(s, dim=1)
    T, k = idx.shape
    ys = []
    for t in range(T):
        yt = torch.zeros(xt.shape[1], dtype=torch.float64)
        for j in range(k):
            if slot[t, j] < 0:
                continue
            e = int(idx[t, j])
            u = W1t[e] @ xt[t]
            if act == oracle.RELU:
                hh = torch.relu(u)
            else:
                hh = torch.nn.functional.silu(u[:F]) * u[F:]
            yt = yt + p[t, e] * (W2t[e] @ hh)
        ys.append(yt)
    y = torch.stack(ys)
    (y * torch.tensor(oracle.to_f64(np.asarray(dy)))).sum().backward()
    g = {"dx": xt.grad.numpy(), "dW1": W1t.grad.numpy(), "dW2": W2t.grad.numpy()}
    if Wgt is not None:
        g["dWg"] = Wgt.grad.numpy()
        g["dbg"] = bgt.grad.numpy() if bgt is not None else None
    return g


@pytest.mark.parametrize("act,normalize,cf,dtype,gate", [
    (oracle.SWIGLU, False, 0.0, "bf16", True),
    (oracle.RELU, False, 0.7, "f32", True),
    (oracle.SWIGLU, True, 1.0, "f32", True),
    (oracle.RELU, True, 0.0, "bf16", False),
])
def test_backward_matches_torch_autograd(act, normalize, cf, dtype, gate):
    T, d, E, k, F = 23, 64, 5, 2, 64
    n1 = 2 * F if act == oracle.SWIGLU else F
    cast = (lambda a: moe_inputs.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    x = cast(RNG.standard_normal((T, d)).astype(np.float32))
    W1 = cast((RNG.standard_normal((E, n1, d)) * 0.1).astype(np.float32))
    W2 = cast((RNG.standard_normal((E, d, F)) * 0.1).astype(np.float32))
    dy = cast(RNG.standard_normal((T, d)).astype(np.float32))
    if gate:
        Wg = cast((RNG.standard_normal((E, d)) * 0.2).astype(np.float32))
        bg = RNG.standard_normal(E).astype(np.float32)
        _ze, z32 = oracle.gate_logits(x, Wg, bg)
    else:
        Wg = bg = None
        z32 = RNG.standard_normal((T, E)).astype(np.float32)
    idx, _w = oracle.route(z32, k, normalize, 1.5)
    disp = oracle.dispatch(idx, E, oracle.capacity(T, E, k, cf))
    g = oracle.backward(x, Wg, W1, W2, z32, idx, disp["slot"], dy, act, F, normalize, 1.5)
    ref = torch_layer_grads(x, Wg, bg, W1, W2, z32, idx, disp["slot"], dy, act, F, normalize, 1.5)
    for name in ("dx", "dW1", "dW2") + (("dWg", "dbg") if gate else ()):
        a, b = g[name], ref[name]
        assert np.allclose(a, b, rtol=1e-10, atol=1e-12 * max(1.0, np.abs(b).max())), name
    if not gate:
        assert not g["dWg"].any() and not g["dbg"].any()


def test_backward_central_differences():
    """d(sum y*dy)/d(param) by central differences of the forward oracle."""
    T, d, E, k, F = 7, 64, 4, 2, 64
    act = oracle.SWIGLU
    x = RNG.standard_normal((T, d)).astype(np.float32)
    Wg = (RNG.standard_normal((E, d)) * 0.3).astype(np.float32)
    bg = (np.arange(E) * 0.5).astype(np.float32)
    W1 = (RNG.standard_normal((E, 2 * F, d)) * 0.1).astype(np.float32)
    W2 = (RNG.standard_normal((E, d, F)) * 0.1).astype(np.float32)
    dy = RNG.standard_normal((T, d)).astype(np.float32)

    def loss(x, Wg, bg, W1, W2):
        out = oracle.moe_forward(x, Wg, bg, W1, W2, k=k, F=F, act=act, normalize_flag=True, lam=0.8)
        return float((out["y"] * dy.astype(np.float64)).sum()), out

    _l0, out0 = loss(x, Wg, bg, W1, W2)
    g = oracle.backward(x, Wg, W1, W2, out0["z32"], out0["topk_idx"], out0["slot"], dy, act, F, True, 0.8)
    checks = [("x", (2, 5), "dx"), ("x", (6, 63), "dx"), ("Wg", (1, 10), "dWg"), ("bg", (3,), "dbg"),
              ("W1", (out0["topk_idx"][0, 0], 3, 7), "dW1"), ("W1", (out0["topk_idx"][1, 1], F + 9, 2), "dW1"),
              ("W2", (out0["topk_idx"][4, 0], 11, 13), "dW2")]
    params = {"x": x, "Wg": Wg, "bg": bg, "W1": W1, "W2": W2}
    for pname, at, gname in checks:
        base = params[pname]
        h = np.float32(2.0 ** -9) * max(1.0, abs(float(base[at])))
        vals = []
        for sgn in (1, -1):
            q = {n: v.copy() for n, v in params.items()}
            q[pname][at] = base[at] + sgn * h
            l, out = loss(**q)
            assert np.array_equal(out["topk_idx"], out0["topk_idx"])  # routing unchanged by the step
            vals.append(l)
        step = float(np.float32(base[at] + h)) - float(np.float32(base[at] - h))
        fd = (vals[0] - vals[1]) / step
        an = g[gname][at]
        assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (pname, at, fd, an)


def test_backward_degenerate_cases():
    T, d, E, k, F = 9, 64, 3, 1, 64
    x = RNG.standard_normal((T, d)).astype(np.float32)
    W1 = (RNG.standard_normal((E, F, d)) * 0.1).astype(np.float32)
    W2 = (RNG.standard_normal((E, d, F)) * 0.1).astype(np.float32)
    Wg = (RNG.standard_normal((E, d)) * 0.1).astype(np.float32)
    dy = RNG.standard_normal((T, d)).astype(np.float32)
    _ze, z32 = oracle.gate_logits(x, Wg, None)
    idx, _ = oracle.route(z32, k)
    # every choice dropped: y == 0 whatever the inputs, so every gradient is 0
    gone = np.full((T, k), -1, np.int32)
    g = oracle.backward(x, Wg, W1, W2, z32, idx, gone, dy, oracle.RELU, F)
    assert not any(g[n].any() for n in ("dx", "dWg", "dbg", "dW1", "dW2"))
    # constant logits under the normalisation: the scores are 0 whatever z, so dz == 0
    zc = np.full((T, E), 0.25, np.float32)
    slot = np.arange(T, dtype=np.int32)[:, None]
    g = oracle.backward(x, None, W1, W2, zc, np.zeros((T, 1), np.int32), slot, dy, oracle.RELU, F, True, 1.0)
    assert not g["dz"].any()
    # a dz row sums to zero: softmax (and the standardisation) are shift invariant
    g = oracle.backward(x, Wg, W1, W2, z32, idx, slot, dy, oracle.RELU, F, True, 2.0)
    assert np.allclose(g["dz"].sum(axis=1), 0.0, atol=1e-12)


@pytest.mark.parametrize("normalize,with_dy", [(False, True), (True, True), (True, False)])
def test_backward_balancing_losses_central_differences(normalize, with_dy):
    """The aux and Z-loss terms of orc_backward against central differences of
    sum(y dy) + a aux + b z_loss, the losses from router_stats (pinned on their
    own above); with dy = 0 the losses alone."""
    T, d, E, k, F = 7, 64, 4, 2, 64
    act = oracle.SWIGLU
    a_coef, b_coef, lam = 0.37, 0.21, 0.8
    x = RNG.standard_normal((T, d)).astype(np.float32)
    Wg = (RNG.standard_normal((E, d)) * 0.3).astype(np.float32)
    bg = (np.arange(E) * 0.5).astype(np.float32)
    W1 = (RNG.standard_normal((E, 2 * F, d)) * 0.1).astype(np.float32)
    W2 = (RNG.standard_normal((E, d, F)) * 0.1).astype(np.float32)
    dy = RNG.standard_normal((T, d)).astype(np.float32) if with_dy else np.zeros((T, d), np.float32)

    def loss(x, Wg, bg, W1, W2):
        out = oracle.moe_forward(x, Wg, bg, W1, W2, k=k, F=F, act=act, normalize_flag=normalize, lam=lam)
        st = oracle.router_stats(out["z32"], out["counts"], out["P"], k, normalize, lam)
        return float((out["y"] * dy.astype(np.float64)).sum() + a_coef * st["aux"] + b_coef * st["z_loss"]), out

    _l0, out0 = loss(x, Wg, bg, W1, W2)
    g = oracle.backward(x, Wg, W1, W2, out0["z32"], out0["topk_idx"], out0["slot"], dy, act, F, normalize, lam,
                        aux_coef=a_coef, z_coef=b_coef)
    checks = [("x", (2, 5), "dx"), ("x", (6, 40), "dx"), ("Wg", (1, 10), "dWg"), ("Wg", (3, 63), "dWg"),
              ("bg", (0,), "dbg"), ("bg", (2,), "dbg")]
    params = {"x": x, "Wg": Wg, "bg": bg, "W1": W1, "W2": W2}
    for pname, at, gname in checks:
        base = params[pname]
        h = np.float32(2.0 ** -9) * max(1.0, abs(float(base[at])))
        vals = []
        for sgn in (1, -1):
            q = {n: v.copy() for n, v in params.items()}
            q[pname][at] = base[at] + sgn * h
            l, out = loss(**q)
            assert np.array_equal(out["topk_idx"], out0["topk_idx"])  # routing unchanged by the step
            vals.append(l)
        step = float(np.float32(base[at] + h)) - float(np.float32(base[at] - h))
        fd = (vals[0] - vals[1]) / step
        an = g[gname][at]
        assert abs(fd - an) <= 2e-3 * max(1e-2, abs(an)), (pname, at, fd, an)
    # the terms are really there: without them the gate gradient differs
    g0 = oracle.backward(x, Wg, W1, W2, out0["z32"], out0["topk_idx"], out0["slot"], dy, act, F, normalize, lam)
    assert np.max(np.abs(g["dWg"] - g0["dWg"])) > 1e-3 * np.max(np.abs(g["dWg"]))
