"""Checks of the seeded synthetic inputs (CPU only)."""
import numpy as np
import pytest

import moe_inputs
import oracle
from _margins import ambiguous_tokens, exact_sum_certified, logit_eps

GATE_CASES = [n for n, c in moe_inputs.CASES.items() if c.logits == "gate"]


def test_generator_is_deterministic_and_per_expert():
    c = moe_inputs.get("mixtral_s")
    a = moe_inputs.make(c)
    b = moe_inputs.make(c, threads=1)
    for key in ("x", "Wg", "bg", "W1", "W2"):
        assert np.array_equal(a[key], b[key]), key
    # expert 3's weights depend only on (seed, tensor, expert)
    w1_3 = moe_inputs.f32_to_bf16_bits(
        moe_inputs.rng(c.seed, moe_inputs.TID_W1, 3).standard_normal((c.n1, c.d), dtype=np.float32)
        * np.float32(c.w_std))
    assert np.array_equal(a["W1"][3], w1_3)


def test_shapes_and_distributions():
    c = moe_inputs.get("tiny_fp32")
    a = moe_inputs.make(c)
    assert a["x"].dtype == np.float32 and a["x"].shape == (256, 64)
    assert a["W1"].shape == (4, 128, 64) and a["W2"].shape == (4, 64, 128)
    assert abs(a["Wg"].std() - 0.125) < 0.01 and abs(a["x"].std() - 0.02) < 0.002
    c = moe_inputs.get("many_small_s")
    a = moe_inputs.make(c, weights=False)
    assert a["logits"].shape == (c.T, c.E) and a["Wg"] is None
    hot_t, hot_e = a["hot_tokens"], a["hot_experts"]
    assert len(hot_t) == round(0.1 * c.T) and len(set(hot_e.tolist())) == 8
    # hot tokens route both choices onto hot experts
    idx, _ = oracle.route(a["logits"], c.k)
    assert np.all(np.isin(idx[hot_t], hot_e))


@pytest.mark.parametrize("name", GATE_CASES)
def test_seeded_gate_cases_have_unambiguous_routing(name):
    """Every fp32 gate logit of these seeded inputs is pinned by the double
    accumulation bound, so the GPU's and the oracle's logits are equal and
    routing from each side's own logits must match bit for bit."""
    case = moe_inputs.get(name)
    inp = moe_inputs.make(case, weights=False)
    z_exact, _ = oracle.gate_logits(inp["x"], inp["Wg"], inp["bg"])
    x64, w64 = oracle.to_f64(inp["x"]), oracle.to_f64(inp["Wg"])
    eps = logit_eps(x64, w64, inp["bg"])
    cert = exact_sum_certified(x64, w64, inp["bg"], 7 if case.dtype == "bf16" else 23)
    amb = ambiguous_tokens(z_exact, eps, cert)
    assert amb.size == 0, f"{name}: ambiguous tokens {amb[:10]}"
