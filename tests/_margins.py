"""When can the GPU's fp32 gate logits differ from the oracle's?

Both sides form z_te = sum_i x_ti Wg_ei (+ bg_e) with the products exact in
double (bf16 x bf16 and fp32 x fp32 products fit in 53 bits) and the sum in
double, then round once to fp32.  A double sum of n exact terms in any order
is within (n - 1) 2^-53 sum|terms| of the exact sum (first order, Higham,
"Accuracy and Stability of Numerical Algorithms", ch. 4); with the bias
term, eps_te = (d + 2) 2^-53 (S_te + |bg_e|), S_te = sum_i |x_ti Wg_ei|.

So both fp32 keys equal round_fp32(v) for some v within eps of the exact sum.
When every value within 2 eps of the oracle's double rounds to the same fp32
number, the two sides' keys are identical and so is every top-k decision taken
on them.  A key for which that fails is "unstable".
"""
import numpy as np

U53 = 2.0 ** -53


def logit_eps(x64, wg64, bg):
    d = x64.shape[1]
    S = np.abs(x64) @ np.abs(wg64).T
    if bg is not None:
        S = S + np.abs(np.asarray(bg, np.float64))[None, :]
    return (d + 2) * U53 * S


def unstable_keys(z_exact, eps):
    """Boolean [T,E]: the fp32 rounding of this logit is not pinned by eps."""
    lo = (z_exact - 2 * eps).astype(np.float32)
    hi = (z_exact + 2 * eps).astype(np.float32)
    return lo != hi


def ambiguous_tokens(z_exact, eps, certified=None):
    """Tokens whose routing could differ between two correct fp32 gates: a key
    that is unstable (and not certified exact) can take either of two adjacent
    fp32 values lo < hi; it can reorder the token's keys only if another key of
    the same token lies in [lo, hi]."""
    bad = unstable_keys(z_exact, eps)
    if certified is not None:
        bad &= ~certified
    out = []
    for t, e in zip(*np.nonzero(bad)):
        lo = np.float32(z_exact[t, e] - 2 * eps[t, e])
        hi = np.float32(z_exact[t, e] + 2 * eps[t, e])
        z32 = z_exact[t].astype(np.float32)
        others = np.delete(z32, e)
        if np.any((others >= lo) & (others <= hi)):
            out.append(t)
    return np.unique(np.array(out, np.int64))


def _lsb_log2(v, mant_bits):
    """log2 of the last significand bit of each nonzero value (normal range);
    -inf for zeros (they add nothing)."""
    a = np.abs(np.asarray(v, np.float64))
    out = np.full(a.shape, -np.inf)
    nz = a > 0
    out[nz] = np.floor(np.log2(a[nz])) - mant_bits
    return out


def exact_sum_certified(x64, wg64, bg, mant_bits, chunk=256):
    """Boolean [T,E]: every partial sum of the terms x_ti Wg_ei (and bg_e), in
    any order, is an integer multiple of the finest term granularity g and at
    most S in magnitude; when S / g < 2^53 each partial sum is a double, so a
    double accumulation in any order returns the exact sum and both sides
    round the same exact value to fp32."""
    T, d = x64.shape
    E = wg64.shape[0]
    lx = _lsb_log2(x64, mant_bits)            # [T,d]
    lw = _lsb_log2(wg64, mant_bits)           # [E,d]
    S = np.abs(x64) @ np.abs(wg64).T
    gmin = np.empty((T, E))
    for t0 in range(0, T, chunk):
        blk = lx[t0:t0 + chunk, None, :] + lw[None, :, :]      # [t,E,d]; -inf for zero terms
        blk = np.where(np.isfinite(blk), blk, np.inf)
        gmin[t0:t0 + chunk] = blk.min(axis=2)
    if bg is not None:
        b = np.asarray(bg, np.float64)
        lb = _lsb_log2(b, 23)
        gmin = np.minimum(gmin, np.where(np.isfinite(lb), lb, np.inf)[None, :])
        S = S + np.abs(b)[None, :]
    with np.errstate(over="ignore"):
        ok = np.log2(np.maximum(S, 1e-300)) - gmin < 53
    return ok | np.isinf(gmin)


# ---------------------------------------------------------------- ReLU backward
# The ReLU backward passes dh where u > 0.  The GPU decides on its stored u:
# an fp32 accumulation of the d products x_ti W1_efi (bf16 products are exact
# in fp32; fp32 products carry one rounding each), then rounded to the storage
# dtype, which keeps the sign.  Any order of fp32 multiply-adds is within
# gamma_{d+1} S of the exact value, gamma_n = n u / (1 - n u), u = 2^-24,
# S = sum_i |x_ti W1_efi| (Higham, ch. 3-4); the bound is doubled as a margin
# for the matrix cores' internal accumulation.  Where |u_exact| is inside that
# bound the two sides may take different, equally correct decisions.
U24 = 2.0 ** -24


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def relu_unpinned(x64, W1, topk_idx, slot, F, d):
    """Triples (t, e, f) of kept choices whose ReLU decision is not pinned
    (x64 [T,d] float64; W1 [E,n1,d] as stored: fp32 or bf16 bits)."""
    n = d + 1
    gamma = 2.0 * n * U24 / (1.0 - n * U24) + (d + 1) * U53
    out = []
    for e in np.unique(topk_idx[slot >= 0]):
        toks = np.nonzero(np.any((topk_idx == e) & (slot >= 0), axis=1))[0]
        xs = x64[toks]
        w = _f64(W1[e, :F])
        u = xs @ w.T
        S = np.abs(xs) @ np.abs(w).T
        bad = np.abs(u) <= gamma * S
        for r, f in zip(*np.nonzero(bad)):
            out.append((int(toks[r]), int(e), int(f)))
    return out
