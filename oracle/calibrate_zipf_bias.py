"""Calibrate the per-expert gate bias of the Zipf-skewed synthetic cases.

Run from the repository root:  python oracle/calibrate_zipf_bias.py [case ...]
(no names: every case; entries of cases not named are kept as stored)

For each case whose gate bias is "zipf", the bias b [E] is chosen so that the
share of top-k assignments that land on expert e follows q_e ~ (e+1)^-s.
Starting from b = 0 it repeats the fixed-point step

    b_e <- b_e + step * sigma_z * (log q_e - log f_e)

(sigma_z: standard deviation of the unbiased logits) where f_e is the
realised share given by the oracle's own routing of the
case's seeded tokens (fp32 logits of x Wg^T + b, top-k by logit).  The result
is written to moe_inputs/zipf_bias.json together with the realised loads.
Only the oracle and the input generator are used.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_inputs  # noqa: E402
import oracle  # noqa: E402

ITERS = 300
STEP = 0.4  # times the standard deviation of the unbiased logits


def calibrate(case):
    inp = moe_inputs.make(case, weights=False, bias_override=np.zeros(case.E, np.float32))
    z_exact, _ = oracle.gate_logits(inp["x"], inp["Wg"], None)
    q = moe_inputs.zipf_shares(case.E, case.zipf_s)
    b = np.zeros(case.E, np.float64)
    step = STEP * float(z_exact.std())
    n_assign = case.T * case.k
    for _ in range(ITERS):
        z32 = (z_exact + b[None, :]).astype(np.float32)
        idx, _w = oracle.route(z32, case.k)
        f = np.bincount(idx.ravel(), minlength=case.E) / n_assign
        f = np.maximum(f, 0.5 / n_assign)
        b += step * (np.log(q) - np.log(f))
        b -= b.mean()
    bias = b.astype(np.float32)
    # realised loads with the stored (fp32) bias, through the oracle's own gate
    _ze, z32 = oracle.gate_logits(inp["x"], inp["Wg"], bias)
    idx, _w = oracle.route(z32, case.k)
    loads = np.bincount(idx.ravel(), minlength=case.E)
    return bias, loads, q


def main():
    table = {}
    if os.path.exists(moe_inputs.ZIPF_BIAS_FILE):
        with open(moe_inputs.ZIPF_BIAS_FILE) as f:
            table = json.load(f)
    names = sys.argv[1:]
    for name, case in moe_inputs.CASES.items():
        if case.bias != "zipf" or (names and name not in names):
            continue
        bias, loads, q = calibrate(case)
        key = moe_inputs.case_key(case)
        table[key] = {
            "case": name,
            "bias": [float(v) for v in bias],
            "realised_loads": [int(v) for v in loads],
            "target_loads": [round(float(v) * case.T * case.k, 1) for v in q],
            "iterations": ITERS,
            "step": STEP,
        }
        print(name, "loads", loads.tolist(), "target", np.round(q * case.T * case.k).astype(int).tolist(), flush=True)
    with open(moe_inputs.ZIPF_BIAS_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
