"""CPU oracle of the sparsely-gated MoE layer forward (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg are the only code that may import this package.
The product path (the HIP library and its Python binding) never imports it,
and this package imports nothing from the product path.

The arithmetic lives in ``moe_oracle.c`` (plain C, double accumulation,
OpenMP over tokens); this module only marshals numpy arrays to it and composes
the steps in the order the layer defines them:

  gate logits -> [normalise] -> softmax -> top-k -> capacity / drop ->
  permutation -> expert FFN -> weighted combine.

Conventions (shared with the HIP path only through the documented layouts):
  * floating tensors are numpy float32 (fp32) or uint16 holding bf16 bits;
  * x [T,d], Wg [E,d], bg [E] fp32, W1 [E,n1,d] (n1 = F or 2F, SwiGLU gate
    rows first), W2 [E,d,F], logits [T,E] fp32;
  * topk_idx [T,k] int32, slot [T,k] int32 (-1 = dropped), counts [E],
    offsets [E+1], src_token [P] int32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1
RELU = 0
SWIGLU = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A sanitizer build of the same source may be loaded instead (host-code
# checks run the pins against it in a child process).
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so (gcc, OpenMP, portable x86-64)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """The same source with AddressSanitizer and UndefinedBehaviorSanitizer
    checks (gcc), for host-code checks of the oracle: load it in a child
    process with gcc's libasan and libubsan preloaded and MOE_ORACLE_LIB=<out>."""
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-o", out, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.orc_threads.restype = I
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_double.restype = D
    lib.orc_gate_logits.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.orc_normalize.argtypes = [I, P, D, P]
    lib.orc_softmax.argtypes = [I, P, P]
    lib.orc_gate_probs.argtypes = [I, P, I, D, P]
    lib.orc_topk.argtypes = [I, I, P, P]
    lib.orc_route.argtypes = [I, I, I, I, D, P, P, P, P]
    lib.orc_capacity.argtypes = [I, I, I, D]
    lib.orc_capacity.restype = ctypes.c_longlong
    lib.orc_dispatch.argtypes = [I, I, I, ctypes.c_longlong, P, P, P, P, P]
    lib.orc_dispatch.restype = I
    lib.orc_expert_ffn.argtypes = [I, I, I, I, P, P, I, P, P, P]
    lib.orc_forward_tokens.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I, P, P]
    lib.orc_ffn_rows.argtypes = [I, I, I, I, I, P, P, P, P, I, P, P, P]
    lib.orc_combine.argtypes = [I, I, I, I, P, P, P, P]
    lib.orc_down_rows.argtypes = [I, I, I, I, P, P, P, I, P, P]
    lib.orc_router_stats.argtypes = [I, I, I, I, D, P, P, ctypes.c_longlong, P, P, P]
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = D
    lib.orc_e4m3_encode.argtypes = [D]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_fp8_scale_exp.argtypes = [D]
    lib.orc_fp8_scale_exp.restype = I
    lib.orc_quant_rows_fp8.argtypes = [ctypes.c_longlong, I, I, P, P, P]
    lib.orc_expert_ffn_fp8.argtypes = [I, I, I, P, P, P, P, I, P, D, P, P]
    lib.orc_ffn_rows_fp8.argtypes = [I, I, I, I, P, P, P, P, P, P, P, I, P, P, P]
    lib.orc_down_rows_fp8.argtypes = [I, I, I, P, P, P, P, P, I, P, P]
    lib.orc_backward.argtypes = [I, I, I, I, I, I, I, I, D, D, D, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.orc_forward_tokens_fp8.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I, P, P]
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle tensors are float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().orc_threads())


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (vectorised, same rule as the C side)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)


def gate_logits(x, Wg, bg=None):
    """z = x Wg^T + bg.  Returns (z_exact float64 [T,E], z32 float32 [T,E])."""
    x = _c(x)
    Wg = _c(Wg)
    T, d = x.shape
    E = Wg.shape[0]
    assert Wg.shape == (E, d) and Wg.dtype == x.dtype
    bgc = None if bg is None else _c(bg, np.float32)
    ze = np.empty((T, E), np.float64)
    z32 = np.empty((T, E), np.float32)
    _load().orc_gate_logits(T, d, E, _dtype_code(x), _ptr(x), _ptr(Wg), _ptr(bgc), _ptr(ze), _ptr(z32))
    return ze, z32


def normalize(z_row, lam):
    z_row = _c(z_row, np.float32)
    E = z_row.shape[0]
    out = np.empty(E, np.float64)
    _load().orc_normalize(E, _ptr(z_row), float(lam), _ptr(out))
    return out


def softmax(s_row):
    s_row = _c(s_row, np.float64)
    E = s_row.shape[0]
    out = np.empty(E, np.float64)
    _load().orc_softmax(E, _ptr(s_row), _ptr(out))
    return out


def gate_probs(z_row, normalize_flag, lam):
    z_row = _c(z_row, np.float32)
    E = z_row.shape[0]
    out = np.empty(E, np.float64)
    _load().orc_gate_probs(E, _ptr(z_row), int(bool(normalize_flag)), float(lam), _ptr(out))
    return out


def topk(z_row, k):
    z_row = _c(z_row, np.float32)
    E = z_row.shape[0]
    out = np.empty(k, np.int32)
    _load().orc_topk(E, k, _ptr(z_row), _ptr(out))
    return out


def route(z32, k, normalize_flag=False, lam=1.0, want_p=False):
    """Routing of all tokens on fp32 logits z32 [T,E].

    Returns (topk_idx int32 [T,k], topk_w float64 [T,k]) and, with want_p,
    also p float64 [T,E]."""
    z32 = _c(z32, np.float32)
    T, E = z32.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    p = np.empty((T, E), np.float64) if want_p else None
    _load().orc_route(T, E, k, int(bool(normalize_flag)), float(lam), _ptr(z32), _ptr(idx), _ptr(w), _ptr(p))
    return (idx, w, p) if want_p else (idx, w)


def capacity(T, E, k, cf) -> int:
    """Expert capacity C = ceil(cf * T * k / E), or -1 for no limit (cf <= 0).

    The capacity factor is a single-precision number (the layer's problem
    statement holds it as fp32), so a Python float is first rounded to the
    nearest fp32 value, and C is the exact ceiling for that value: fp32(0.3)
    is slightly above 0.3, so T*k/E = 100 gives C = 31 (a dyadic factor such
    as 0.25 or 1.25 lands on integers exactly).  The C routine evaluates the
    product and quotient in double, which is exact here (a 24-bit factor times
    T*k < 2^27 fits in 53 bits, and a quotient that is not an integer lies
    further from one than a double rounding can move it)."""
    return int(_load().orc_capacity(int(T), int(E), int(k), float(np.float32(cf))))


def dispatch(topk_idx, E, C):
    """Counting + capacity + permutation.  Returns dict of counts, offsets,
    slot, src_token (length P) and P."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    slot = np.empty((T, k), np.int32)
    src = np.full(T * k, -1, np.int32)
    P = _load().orc_dispatch(T, E, k, int(C), _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(slot), _ptr(src))
    return {"counts": counts, "offsets": offsets, "slot": slot, "src_token": src[:P].copy(), "P": int(P)}


def expert_ffn(W1, W2, e, x_row, act, F, want_h=False):
    """One input vector (float64 [d]) through expert e."""
    W1 = _c(W1)
    W2 = _c(W2)
    d = W2.shape[1]
    xr = _c(x_row, np.float64)
    out = np.empty(d, np.float64)
    h = np.empty(F, np.float64) if want_h else None
    _load().orc_expert_ffn(d, F, int(act), _dtype_code(W1), _ptr(W1), _ptr(W2), int(e), _ptr(xr), _ptr(out), _ptr(h))
    return (out, h) if want_h else out


def forward_tokens(x, W1, W2, topk_idx, topk_w, slot, act, F, tokens=None):
    """Layer output rows (float64 [n, d]) for the given tokens (default all)."""
    x = _c(x)
    W1 = _c(W1)
    W2 = _c(W2)
    T, d = x.shape
    idx = _c(topk_idx, np.int32)
    k = idx.shape[1]
    w = _c(topk_w, np.float64)
    sl = _c(slot, np.int32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tok is None else tok.shape[0]
    y = np.empty((n, d), np.float64)
    _load().orc_forward_tokens(d, k, F, int(act), _dtype_code(x), _ptr(x), _ptr(W1), _ptr(W2), _ptr(idx), _ptr(w),
                               _ptr(sl), n, _ptr(tok), _ptr(y))
    return y


def ffn_rows(x_perm, offsets, W1, W2, act, F, rows=None, want_h=False):
    """Expert FFN of permuted rows (float64 [n, d]); the expert of a row is
    found from offsets."""
    xp = _c(x_perm)
    W1 = _c(W1)
    W2 = _c(W2)
    off = _c(offsets, np.int32)
    E = off.shape[0] - 1
    d = W2.shape[1]
    rr = None if rows is None else _c(rows, np.int32)
    n = xp.shape[0] if rr is None else rr.shape[0]
    out = np.empty((n, d), np.float64)
    h = np.empty((n, F), np.float64) if want_h else None
    _load().orc_ffn_rows(E, d, F, int(act), _dtype_code(xp), _ptr(off), _ptr(xp), _ptr(W1), _ptr(W2), n, _ptr(rr),
                         _ptr(out), _ptr(h))
    return (out, h) if want_h else out


def down_rows(h, offsets, W2, rows=None):
    """Second expert layer on given hidden rows h [*, F] (float64 [n, d])."""
    h = _c(h)
    W2 = _c(W2)
    off = _c(offsets, np.int32)
    E = off.shape[0] - 1
    d, F = W2.shape[1], W2.shape[2]
    rr = None if rows is None else _c(rows, np.int32)
    n = h.shape[0] if rr is None else rr.shape[0]
    out = np.empty((n, d), np.float64)
    _load().orc_down_rows(E, d, F, _dtype_code(h), _ptr(off), _ptr(h), _ptr(W2), n, _ptr(rr), _ptr(out))
    return out


def combine(y_perm, slot, topk_w, T):
    yp = _c(y_perm)
    sl = _c(slot, np.int32)
    w = _c(topk_w, np.float64)
    k = sl.shape[1]
    d = yp.shape[1]
    y = np.empty((T, d), np.float64)
    _load().orc_combine(T, d, k, _dtype_code(yp), _ptr(yp), _ptr(sl), _ptr(w), _ptr(y))
    return y


def moe_forward(x, Wg, bg, W1, W2, *, k, F, act, normalize_flag=False, lam=1.0, cf=0.0, logits=None,
                tokens=None):
    """Whole layer, composed step by step.  When logits (fp32 [T,E]) is given,
    the gate is skipped and those logits are routed.  Returns a dict with the
    routing, the permutation and y (float64) for the requested tokens."""
    x = _c(x)
    T = x.shape[0]
    if logits is None:
        z_exact, z32 = gate_logits(x, Wg, bg)
    else:
        z32 = _c(logits, np.float32)
        z_exact = None
    E = z32.shape[1]
    idx, w = route(z32, k, normalize_flag, lam)
    C = capacity(T, E, k, cf)
    disp = dispatch(idx, E, C)
    y = forward_tokens(x, W1, W2, idx, w, disp["slot"], act, F, tokens)
    out = {"z_exact": z_exact, "z32": z32, "topk_idx": idx, "topk_w": w, "C": C, "y": y}
    out.update(disp)
    return out


def router_stats(z32, counts, kept, k, normalize_flag=False, lam=1.0):
    """Router by-products of a routed batch (see orc_router_stats): a dict
    with frac [E], mean_prob [E] and the scalars aux, z_loss, drop_rate, all
    float64.  z32 are the fp32 logits the routing used, counts the per-expert
    assignment counts before the capacity clip, kept the assignments kept."""
    z = _c(z32, np.float32)
    T, E = z.shape
    cnt = _c(counts, np.int32)
    frac = np.empty(E, np.float64)
    mp = np.empty(E, np.float64)
    out3 = np.empty(3, np.float64)
    _load().orc_router_stats(T, E, int(k), int(bool(normalize_flag)), float(lam), _ptr(z), _ptr(cnt), int(kept),
                             _ptr(frac), _ptr(mp), _ptr(out3))
    return {"frac": frac, "mean_prob": mp, "aux": out3[0], "z_loss": out3[1], "drop_rate": out3[2]}


def shared_expert(x, Ws1, Ws2, act, Fs):
    """Shared expert: one more expert FFN that every token passes through,
    ungated (industry overview page, "MoE未來重點研究方向" item 4: DeepSeekMoE's
    shared experts).  x [T,d]; Ws1 [n1,d] (SwiGLU gate rows first), Ws2 [d,Fs].
    It is the expert FFN of a single expert whose segment holds all T rows.
    Returns float64 [T,d]."""
    x = _c(x)
    T = x.shape[0]
    offsets = np.array([0, T], np.int32)
    return ffn_rows(x, offsets, np.asarray(Ws1)[None], np.asarray(Ws2)[None], act, Fs)


def combine_shared(y_perm, slot, topk_w, y_shared):
    """Combine with a shared expert: y[t] = y_shared[t] + sum over the kept
    choices j of w[t,j] * y_perm[slot[t,j]] (the shared expert's output enters
    with weight one).  y_shared is float64 or a stored fp32/bf16 array."""
    ys = to_f64(np.asarray(y_shared)) if np.asarray(y_shared).dtype != np.float64 else np.asarray(y_shared)
    return ys + combine(y_perm, slot, topk_w, ys.shape[0])


# ---------------------------------------------------------------- FP8 (E4M3)
# Expert weights and activations as OCP FP8 E4M3 codes with power-of-two row
# scales (see the FP8 entry of moe_oracle.c's header for the reading).

def e4m3_decode(codes):
    """Values (float64) of E4M3 codes (uint8 array)."""
    c = np.asarray(codes, np.uint8)
    lib = _load()
    table = np.array([lib.orc_e4m3_decode(i) for i in range(256)], np.float64)
    return table[c]


def e4m3_encode(values):
    """Nearest E4M3 codes (ties to even, saturating at 448) of finite values."""
    v = np.asarray(values, np.float64)
    lib = _load()
    out = np.empty(v.shape, np.uint8)
    flat_in, flat_out = v.ravel(), out.ravel()
    for i in range(flat_in.size):
        flat_out[i] = lib.orc_e4m3_encode(float(flat_in[i]))
    return out


def fp8_scale_exp(amax):
    return _load().orc_fp8_scale_exp(float(amax))


def quant_rows_fp8(src):
    """Per-row power-of-two quantisation of a [R, K] array (float32, uint16
    bf16 bits or float64): returns (codes uint8 [R, K], scales float32 [R])."""
    a = np.asarray(src)
    if a.dtype == np.float64:
        a = np.ascontiguousarray(a)
        code = 2
    else:
        a = _c(a)
        code = _dtype_code(a)
    R, K = a.shape
    codes = np.empty((R, K), np.uint8)
    scales = np.empty(R, np.float32)
    _load().orc_quant_rows_fp8(R, K, code, _ptr(a), _ptr(codes), _ptr(scales))
    return codes, scales


def ffn_rows_fp8(xq, xs, offsets, W1q, w1s, W2q, w2s, act, F, rows=None, want_h=False):
    """FP8 expert FFN of permuted quantised rows (float64 [n, d]); h, when
    asked for, is the activation output before its quantisation."""
    xq = np.ascontiguousarray(xq, np.uint8)
    xs = np.ascontiguousarray(xs, np.float32)
    W1q = np.ascontiguousarray(W1q, np.uint8)
    W2q = np.ascontiguousarray(W2q, np.uint8)
    w1s = np.ascontiguousarray(w1s, np.float32)
    w2s = np.ascontiguousarray(w2s, np.float32)
    off = _c(offsets, np.int32)
    E = off.shape[0] - 1
    d = W2q.shape[1]
    rr = None if rows is None else _c(rows, np.int32)
    n = xq.shape[0] if rr is None else rr.shape[0]
    out = np.empty((n, d), np.float64)
    h = np.empty((n, F), np.float64) if want_h else None
    _load().orc_ffn_rows_fp8(E, d, F, int(act), _ptr(off), _ptr(xq), _ptr(xs), _ptr(W1q), _ptr(w1s), _ptr(W2q),
                             _ptr(w2s), n, _ptr(rr), _ptr(out), _ptr(h))
    return (out, h) if want_h else out


def down_rows_fp8(hq, hs, offsets, W2q, w2s, rows=None):
    """Second FP8 layer on given quantised hidden rows (float64 [n, d])."""
    hq = np.ascontiguousarray(hq, np.uint8)
    hs = np.ascontiguousarray(hs, np.float32)
    W2q = np.ascontiguousarray(W2q, np.uint8)
    w2s = np.ascontiguousarray(w2s, np.float32)
    off = _c(offsets, np.int32)
    E = off.shape[0] - 1
    d, F = W2q.shape[1], W2q.shape[2]
    rr = None if rows is None else _c(rows, np.int32)
    n = hq.shape[0] if rr is None else rr.shape[0]
    out = np.empty((n, d), np.float64)
    _load().orc_down_rows_fp8(E, d, F, _ptr(off), _ptr(hq), _ptr(hs), _ptr(W2q), _ptr(w2s), n, _ptr(rr), _ptr(out))
    return out


def forward_tokens_fp8(x, W1q, w1s, W2q, w2s, topk_idx, topk_w, slot, act, F, tokens=None):
    """FP8 layer output rows (float64 [n, d]) for the given tokens."""
    x = _c(x)
    T, d = x.shape
    W1q = np.ascontiguousarray(W1q, np.uint8)
    W2q = np.ascontiguousarray(W2q, np.uint8)
    w1s = np.ascontiguousarray(w1s, np.float32)
    w2s = np.ascontiguousarray(w2s, np.float32)
    idx = _c(topk_idx, np.int32)
    k = idx.shape[1]
    w = _c(topk_w, np.float64)
    sl = _c(slot, np.int32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tok is None else tok.shape[0]
    y = np.empty((n, d), np.float64)
    _load().orc_forward_tokens_fp8(d, k, F, int(act), _dtype_code(x), _ptr(x), _ptr(W1q), _ptr(w1s), _ptr(W2q),
                                   _ptr(w2s), _ptr(idx), _ptr(w), _ptr(sl), n, _ptr(tok), _ptr(y))
    return y


def quant_weights_fp8(W):
    """E4M3 codes and per-row scales of an expert weight stack [E, rows, K]."""
    W = np.asarray(W)
    E, R, K = W.shape
    codes, scales = quant_rows_fp8(W.reshape(E * R, K))
    return codes.reshape(E, R, K), scales.reshape(E, R)


# ---------------------------------------------------------------- backward
def backward(x, Wg, W1, W2, z32, topk_idx, slot, dy, act, F, normalize_flag=False, lam=1.0, aux_coef=0.0,
             z_coef=0.0):
    """Gradient of the layer (see orc_backward): dict of float64 dx [T,d], dWg
    [E,d], dbg [E], dW1 [E,n1,d], dW2 [E,d,F], dz [T,E].  Wg None means the
    logits were given: dWg and dbg come back as zeros and dx has no gate term.
    aux_coef, z_coef: the balancing losses of router_stats added to the loss."""
    x = _c(x)
    T, d = x.shape
    W1 = _c(W1)
    W2 = _c(W2)
    E, n1 = W1.shape[0], W1.shape[1]
    z = _c(z32, np.float32)
    idx = _c(topk_idx, np.int32)
    k = idx.shape[1]
    sl = _c(slot, np.int32)
    dyc = _c(dy)
    if _dtype_code(dyc) != _dtype_code(x):
        raise TypeError("dy must have the dtype of x")
    Wgc = None if Wg is None else _c(Wg)
    out = {"dx": np.empty((T, d)), "dWg": np.empty((E, d)), "dbg": np.empty(E), "dW1": np.empty((E, n1, d)),
           "dW2": np.empty((E, d, F)), "dz": np.empty((T, E))}
    _load().orc_backward(T, d, E, k, F, int(act), _dtype_code(x), int(bool(normalize_flag)), float(lam),
                         float(aux_coef), float(z_coef), _ptr(x),
                         _ptr(Wgc), _ptr(W1), _ptr(W2), _ptr(z), _ptr(idx), _ptr(sl), _ptr(dyc), _ptr(out["dx"]),
                         _ptr(out["dWg"]), _ptr(out["dbg"]), _ptr(out["dW1"]), _ptr(out["dW2"]), _ptr(out["dz"]))
    return out
