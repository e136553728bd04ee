"""Derived error allowance of the FP8 (E4M3) layer against the oracle.

The GPU quantises its own bf16 h, within 2^-9 (one bf16 rounding) plus 2^-16
(fp32 arithmetic, far below it) relative of the exact h, while the oracle
quantises the exact h.  A code of h can differ only where
[|v|(1 - rel), |v|(1 + rel)] (v = h / 2^e in the row's scale) holds a rounding
midpoint of the E4M3 grid; it then moves by at most the gap between the two
neighbouring codes, times the row scale.  A row whose scale exponent itself
is ambiguous gets twice the coarser gap on every element.  The change reaches
y[t] through w_j |W2| (dequantised).  Everything here is the oracle's (its
exact h and its codes); the GPU's outputs are not read."""
import numpy as np

import oracle


def fp8_code_allowance(case, x, W1q, w1s, W2q, w2s, w, disp, tokens=None):
    """Per-token allowance, [T, d] (or [len(tokens), d] for a token subset;
    only the permuted rows of those tokens are evaluated)."""
    act = oracle.SWIGLU if case.act == "swiglu" else oracle.RELU
    xq, xs = oracle.quant_rows_fp8(x)
    src, slot, offs = disp["src_token"], disp["slot"], disp["offsets"]
    F, d, E = case.F, case.d, case.E
    toks = np.arange(case.T) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(toks), d))
    rows = np.unique(slot[toks][slot[toks] >= 0])
    if rows.size == 0:
        return out
    # the chosen rows keep their expert order; sub-offsets per expert
    sub_off = np.searchsorted(rows, offs).astype(np.int32)
    _, h = oracle.ffn_rows_fp8(xq[src[rows]], xs[src[rows]], sub_off, W1q, w1s, W2q, w2s, act, F, want_h=True)
    grid = np.abs(oracle.e4m3_decode(np.arange(128, dtype=np.uint8)))
    mags = np.unique(grid[np.isfinite(grid)])  # the grid, 0 .. 448 (the NaN code left out)
    mids = (mags[1:] + mags[:-1]) / 2
    gaps = mags[1:] - mags[:-1]
    rel = 2.0 ** -9 + 2.0 ** -16
    amax = np.max(np.abs(h), axis=1)
    e = np.array([oracle.fp8_scale_exp(a) for a in amax])
    ambiguous = np.array([oracle.fp8_scale_exp(a * (1 - rel)) != oracle.fp8_scale_exp(a * (1 + rel)) for a in amax])
    s = 2.0 ** e
    a = np.abs(h) / s[:, None]
    lo = np.searchsorted(mids, a * (1 - rel), side="left")
    hi = np.searchsorted(mids, a * (1 + rel), side="right")
    coef = np.where(hi > lo, gaps[np.minimum(lo, gaps.size - 1)], 0.0) * s[:, None]
    coarse = gaps[np.minimum(np.searchsorted(mids, a), gaps.size - 1)] * s[:, None] * 2
    coef[ambiguous] = 2 * coarse[ambiguous]
    per_row = np.zeros((rows.size, d))
    for ex in range(E):
        r0, r1 = sub_off[ex], sub_off[ex + 1]
        if r1 > r0:
            W2d = np.abs(oracle.e4m3_decode(W2q[ex]) * np.asarray(w2s[ex], np.float64)[:, None])  # [d, F]
            per_row[r0:r1] = coef[r0:r1] @ W2d.T
    where = {int(r): i for i, r in enumerate(rows)}
    for i, t in enumerate(toks):
        for j in range(case.k):
            r = slot[t, j]
            if r >= 0:
                out[i] += w[t, j] * per_row[where[int(r)]]
    return out
