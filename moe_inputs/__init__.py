"""Seeded synthetic inputs for the MoE-layer forward.

This module is the only code shared by the HIP path's tests/benchmark and the
CPU oracle.  It draws random tensors and lays them out; it holds none of the
layer's arithmetic (no gate, routing, permutation or FFN).

Random streams: every (case seed, tensor id, expert) triple has its own
``numpy.random.Generator(PCG64(SeedSequence([seed, tensor, expert])))``, so
a weight tensor is reproducible expert by expert and can be drawn in
parallel.  Values are drawn in float32 from N(0, std^2) and, for bf16 cases,
rounded to bf16 with round-to-nearest-even (stored as uint16 bit patterns).

The per-expert gate bias of the Zipf-skewed cases is an input too.  It is
calibrated by ``oracle/calibrate_zipf_bias.py`` (which runs the oracle's
routing on these very inputs) and stored in ``zipf_bias.json`` beside this
file; this module only reads it.
"""
from __future__ import annotations

import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
ZIPF_BIAS_FILE = os.path.join(_HERE, "zipf_bias.json")

# tensor ids for the seed sequence
TID_X, TID_WG, TID_W1, TID_W2, TID_LOGITS, TID_HOT, TID_DY = 1, 2, 3, 4, 5, 6, 7


@dataclass(frozen=True)
class Case:
    """One synthetic workload: shapes, layer options and input distributions."""
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    act: str                  # "relu" | "swiglu"
    dtype: str                # "f32" | "bf16"
    seed: int
    normalize: bool = False   # Skywork gating-logit normalisation
    lam: float = 1.0
    cf: float = 0.0           # capacity factor; <= 0 is dropless
    logits: str = "gate"      # "gate": logits from x Wg^T + bg; "given": drawn directly
    x_std: float = 1.0
    w_std: float = 0.02       # W1, W2
    wg_std: float = 0.02      # gate weight
    bias: str = "none"        # "none" | "zipf" (calibrated per-expert gate bias)
    zipf_s: float = 1.2
    hot_frac: float = 0.0     # given logits: fraction of tokens pushed onto hot experts
    hot_experts: int = 0
    hot_boost: float = 0.0

    @property
    def n1(self) -> int:
        return 2 * self.F if self.act == "swiglu" else self.F

    @property
    def ffn_flops_dropless(self) -> int:
        per_row = 2 * self.d * self.n1 + 2 * self.F * self.d
        return self.T * self.k * per_row

    def with_(self, **kw) -> "Case":
        return replace(self, **kw)


# The five workloads of the layer, at their full sizes.
FULL = {
    # Tiny fp32 layer: T=256, d=64, E=4, top-2, 64->128->64 ReLU, plain softmax gate,
    # no capacity; tokens and expert weights N(0, 0.02^2), gate weights N(0, 1/d).
    "tiny_fp32": Case("tiny_fp32", T=256, d=64, E=4, k=2, F=128, act="relu", dtype="f32", seed=1001,
                      x_std=0.02, w_std=0.02, wg_std=1.0 / math.sqrt(64)),
    # FastMoE Transformer-XL-shaped layer: 64 experts top-2, 512->1024->512 ReLU.
    "fastmoe_txl": Case("fastmoe_txl", T=8192, d=512, E=64, k=2, F=1024, act="relu", dtype="bf16", seed=1002),
    # Mixtral-8x7B-shaped layer, SwiGLU 4096->14336->4096, gate bias giving Zipf(1.2) loads.
    "mixtral": Case("mixtral", T=4096, d=4096, E=8, k=2, F=14336, act="swiglu", dtype="bf16", seed=1003,
                    bias="zipf"),
    # Skywork-MoE-Medium-shaped layer, 16 experts top-2, SwiGLU 4608->12288->4608,
    # gating-logit normalisation lambda = 1, capacity factor 1.25.
    "skywork_m": Case("skywork_m", T=4096, d=4608, E=16, k=2, F=12288, act="swiglu", dtype="bf16", seed=1004,
                      normalize=True, lam=1.0, cf=1.25),
    # Many small experts: 512 experts top-2, ReLU 1024->512->1024, logits N(0,1) given,
    # 10% of tokens pushed onto 8 hot experts.
    "many_small": Case("many_small", T=16384, d=1024, E=512, k=2, F=512, act="relu", dtype="bf16", seed=1005,
                       logits="given", hot_frac=0.10, hot_experts=8, hot_boost=8.0),
}

# A Skywork-shaped variant whose Zipf-skewed gate makes the capacity limit bite.
FULL["skywork_m_zipf"] = FULL["skywork_m"].with_(name="skywork_m_zipf", seed=1014, bias="zipf")

# Reduced cases of the same families, small enough for the oracle to check
# every output in seconds, still spanning several GEMM tiles with ragged tails.
SMALL = {
    "tiny_fp32": FULL["tiny_fp32"],
    "fastmoe_txl_s": FULL["fastmoe_txl"].with_(name="fastmoe_txl_s", T=1024, seed=2002),
    "mixtral_s": FULL["mixtral"].with_(name="mixtral_s", T=600, d=256, F=448, seed=2003),
    "skywork_m_s": FULL["skywork_m"].with_(name="skywork_m_s", T=512, d=320, F=384, seed=2004),
    "skywork_m_zipf_s": FULL["skywork_m_zipf"].with_(name="skywork_m_zipf_s", T=512, d=320, F=384, seed=2014),
    "many_small_s": FULL["many_small"].with_(name="many_small_s", T=2048, d=256, F=128, seed=2005),
    # Mixtral-family layers with about 680 rows per expert, so that the
    # expert GEMMs take their largest (256 x 256) tile and the whole layer is
    # still checked output by output: Zipf(1.2) loads, dropless and with a
    # capacity factor of 1 that clips the two hottest experts.
    "mixtral_m": FULL["mixtral"].with_(name="mixtral_m", T=2048, d=512, E=6, F=768, seed=2006),
    "mixtral_m_cap": FULL["mixtral"].with_(name="mixtral_m_cap", T=2048, d=512, E=6, F=768, seed=2007, cf=1.0),
    # A FastMoE-family layer with 256 rows per expert and a 1024-wide hidden
    # layer: its down-projection (K = 1024) takes the 256 x 256 tile, its
    # up-projection (K = 256) the 128 x 128 one.
    "fastmoe_m": FULL["fastmoe_txl"].with_(name="fastmoe_m", T=2048, d=256, E=16, seed=2008),
}

# Large token counts at small widths: index arithmetic, grids and chunk loops
# at about a million routed rows (routing, permutation, combine) and at a
# quarter million for the backward (long K ranges of the weight gradients,
# many gate-gradient chunks).
LARGE = {
    "large_t_fwd": Case("large_t_fwd", T=(1 << 20) + 13, d=64, E=64, k=2, F=64, act="relu", dtype="bf16",
                        seed=3001, cf=1.0, logits="given"),
    "large_t_bwd": Case("large_t_bwd", T=(1 << 18) + 7, d=64, E=16, k=2, F=64, act="swiglu", dtype="bf16",
                        seed=3002, cf=1.25, normalize=True),
}

CASES = dict(FULL)
CASES.update(SMALL)
CASES.update(LARGE)


def get(name: str) -> Case:
    return CASES[name]


def rng(seed: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, expert])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits.
    Inputs here are finite normal draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed, tensor, expert, shape, std) -> np.ndarray:
    g = rng(seed, tensor, expert)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    return a if dtype == "f32" else f32_to_bf16_bits(a)


def _expert_stack(case: Case, tensor: int, rows: int, cols: int, std: float, threads: int) -> np.ndarray:
    out_dtype = np.float32 if case.dtype == "f32" else np.uint16
    out = np.empty((case.E, rows, cols), out_dtype)

    def one(e):
        out[e] = _cast(_normal(case.seed, tensor, e, (rows, cols), std), case.dtype)

    if threads > 1 and case.E > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(case.E)))
    else:
        for e in range(case.E):
            one(e)
    return out


def zipf_bias(case: Case) -> np.ndarray:
    """Stored calibrated gate bias (float32 [E]) of a Zipf-skewed case."""
    if not os.path.exists(ZIPF_BIAS_FILE):
        raise FileNotFoundError(f"{ZIPF_BIAS_FILE} missing: run oracle/calibrate_zipf_bias.py")
    with open(ZIPF_BIAS_FILE) as f:
        table = json.load(f)
    key = case_key(case)
    if key not in table:
        raise KeyError(f"no calibrated Zipf bias for {key}: run oracle/calibrate_zipf_bias.py")
    return np.array(table[key]["bias"], dtype=np.float32)


def case_key(case: Case) -> str:
    return f"{case.name}:T{case.T}:d{case.d}:E{case.E}:k{case.k}:seed{case.seed}:s{case.zipf_s}"


def make(case, *, weights: bool = True, threads: int = 8, bias_override=None) -> dict:
    """Draw every input tensor of a case (host numpy arrays).

    Returns dict with x [T,d], Wg [E,d] or None, bg [E] float32 or None,
    logits [T,E] float32 or None (given-logits cases), W1 [E,n1,d], W2 [E,d,F]
    (omitted when weights=False)."""
    if isinstance(case, str):
        case = get(case)
    out = {"case": case}
    out["x"] = _cast(_normal(case.seed, TID_X, 0, (case.T, case.d), case.x_std), case.dtype)
    if case.logits == "gate":
        out["Wg"] = _cast(_normal(case.seed, TID_WG, 0, (case.E, case.d), case.wg_std), case.dtype)
        out["logits"] = None
        if bias_override is not None:
            out["bg"] = np.asarray(bias_override, dtype=np.float32)
        elif case.bias == "zipf":
            out["bg"] = zipf_bias(case)
        else:
            out["bg"] = None
    else:
        z = _normal(case.seed, TID_LOGITS, 0, (case.T, case.E), 1.0)
        if case.hot_frac > 0 and case.hot_experts > 0:
            g = rng(case.seed, TID_HOT, 0)
            n_hot_tok = int(round(case.hot_frac * case.T))
            toks = g.choice(case.T, size=n_hot_tok, replace=False)
            hot = g.choice(case.E, size=case.hot_experts, replace=False)
            z[np.ix_(toks, hot)] += np.float32(case.hot_boost)
            out["hot_tokens"] = np.sort(toks).astype(np.int32)
            out["hot_experts"] = np.sort(hot).astype(np.int32)
        out["logits"] = z
        out["Wg"] = None
        out["bg"] = None
    if weights:
        out["W1"] = _expert_stack(case, TID_W1, case.n1, case.d, case.w_std, threads)
        out["W2"] = _expert_stack(case, TID_W2, case.d, case.F, case.w_std, threads)
    return out


def make_dy(case, tokens=None, std: float = 1.0) -> np.ndarray:
    """Incoming gradient dL/dy [T,d] of the backward, N(0, std^2) in the case's
    dtype; with ``tokens`` (indices), rows outside them are zero."""
    if isinstance(case, str):
        case = get(case)
    dy = _normal(case.seed, TID_DY, 0, (case.T, case.d), std)
    if tokens is not None:
        keep = np.zeros(case.T, bool)
        keep[np.asarray(tokens)] = True
        dy[~keep] = 0.0
    return _cast(dy, case.dtype)


def zipf_shares(E: int, s: float) -> np.ndarray:
    """Target assignment shares q_e proportional to (e+1)^-s."""
    q = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return q / q.sum()
