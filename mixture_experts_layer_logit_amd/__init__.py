"""MI355X (gfx950) MoE-layer forward: Python binding of libmoe.so.

The binding only marshals arguments: every step of the layer runs in the HIP
kernels behind the C ABI of ``include/moe.h``.  Torch tensors provide device
memory and the current HIP stream; there is no CPU or PyTorch fallback, and
loading fails loudly when the library has not been built.

Entry points (same names as the C ABI): moe_capacity, moe_workspace_size,
moe_route, moe_permute, moe_expert_up, moe_expert_down, moe_grouped_ffn,
moe_combine, moe_forward, moe_router_stats, moe_shared_workspace_size,
moe_shared_expert, moe_combine_shared, moe_quantize_fp8, moe_fp8_workspace_size,
moe_expert_up_fp8, moe_expert_down_fp8, moe_forward_fp8, moe_forward_train,
moe_backward_workspace_size, moe_backward, moe_forward_noalloc.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB names another build of the same sources (the host-sanitizer build)
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_ACT_RELU, MOE_ACT_SWIGLU = 0, 1
MOE_F32, MOE_BF16 = 0, 1

EXPORTS = ("moe_status_string", "moe_last_error", "moe_capacity", "moe_workspace_size", "moe_route",
           "moe_permute", "moe_expert_up", "moe_expert_down", "moe_grouped_ffn", "moe_combine", "moe_forward",
           "moe_router_stats", "moe_shared_workspace_size", "moe_shared_expert", "moe_combine_shared",
           "moe_quantize_fp8", "moe_fp8_workspace_size", "moe_expert_up_fp8", "moe_expert_down_fp8",
           "moe_forward_fp8", "moe_forward_train", "moe_backward_workspace_size", "moe_backward",
           "moe_forward_noalloc")


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("F", ctypes.c_int32), ("act", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("normalize", ctypes.c_int32), ("lambda_", ctypes.c_float), ("capacity_factor", ctypes.c_float)]


class RouteInfo(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("slot", ctypes.c_void_p), ("src_token", ctypes.c_void_p)]


class RouterLosses(ctypes.Structure):
    _fields_ = [("aux_coef", ctypes.c_float), ("z_coef", ctypes.c_float)]


class Saved(ctypes.Structure):
    _fields_ = [("u", ctypes.c_void_p), ("h", ctypes.c_void_p), ("y_perm", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m mixture_experts_layer_logit_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(Problem)
    st = ctypes.c_int
    lib.moe_status_string.argtypes = [st]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_capacity.argtypes = [PP, ctypes.POINTER(ctypes.c_int32)]
    lib.moe_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_route.argtypes = [PP, P, P, P, P, P, P, P]
    lib.moe_permute.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_expert_up.argtypes = [PP, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_expert_down.argtypes = [PP, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_grouped_ffn.argtypes = [PP, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_combine.argtypes = [PP, P, P, P, P, P]
    lib.moe_forward.argtypes = [PP, P, P, P, P, P, P, P, ctypes.POINTER(RouteInfo), P, ctypes.c_size_t, P]
    lib.moe_forward_noalloc.argtypes = [PP, P, P, P, P, P, P, P, ctypes.POINTER(RouteInfo), P]
    lib.moe_router_stats.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_shared_workspace_size.argtypes = [PP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_shared_expert.argtypes = [PP, ctypes.c_int32, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_combine_shared.argtypes = [PP, P, P, P, P, P, P]
    lib.moe_quantize_fp8.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P, P]
    lib.moe_fp8_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_expert_up_fp8.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_expert_down_fp8.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_forward_fp8.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.POINTER(RouteInfo), P, ctypes.c_size_t,
                                    P]
    lib.moe_forward_train.argtypes = [PP, P, P, P, P, P, P, P, ctypes.POINTER(RouteInfo), ctypes.POINTER(Saved), P,
                                      ctypes.c_size_t, P]
    lib.moe_backward_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_backward.argtypes = [PP, P, P, P, P, P, P, ctypes.POINTER(RouteInfo), ctypes.POINTER(Saved),
                                 ctypes.POINTER(RouterLosses), P, P, P, P, P, P, ctypes.c_size_t, P]
    for name in EXPORTS[2:]:
        getattr(lib, name).restype = st
    _lib = lib
    return lib


def status_name(status: int) -> str:
    try:
        return load().moe_status_string(status).decode()
    except ImportError:
        return str(status)


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, load().moe_last_error().decode())


def problem(T, d, E, k, F, act="relu", dtype="bf16", normalize=False, lam=1.0, cf=0.0) -> Problem:
    """Build the moe_problem struct (act: "relu"|"swiglu", dtype: "f32"|"bf16")."""
    a = {"relu": MOE_ACT_RELU, "swiglu": MOE_ACT_SWIGLU}.get(act, act)
    t = {"f32": MOE_F32, "bf16": MOE_BF16}.get(dtype, dtype)
    return Problem(int(T), int(d), int(E), int(k), int(F), int(a), int(t), int(bool(normalize)), float(lam),
                   float(cf))


def _ptr(t):
    """Device address of a tensor (None -> NULL); plain ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def moe_capacity(p: Problem) -> int:
    c = ctypes.c_int32()
    _check(load().moe_capacity(ctypes.byref(p), ctypes.byref(c)))
    return c.value


def moe_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check(load().moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def _nbytes(ws):
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def moe_route(p, x, Wg, bg, logits, topk_idx, topk_w, stream=None):
    _check(load().moe_route(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(logits), _ptr(topk_idx),
                            _ptr(topk_w), _stream(stream)))


def moe_permute(p, topk_idx, x, counts, offsets, slot, src_token, x_perm, ws, stream=None):
    _check(load().moe_permute(ctypes.byref(p), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets), _ptr(slot),
                              _ptr(src_token), _ptr(x_perm), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_expert_up(p, a, src_token, offsets, W1, h, ws=None, stream=None):
    """a is x_perm (src_token None) or x (rows gathered through src_token)."""
    _check(load().moe_expert_up(ctypes.byref(p), _ptr(a), _ptr(src_token), _ptr(offsets), _ptr(W1), _ptr(h),
                                _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_expert_down(p, h, offsets, W2, y_perm, ws=None, stream=None):
    _check(load().moe_expert_down(ctypes.byref(p), _ptr(h), _ptr(offsets), _ptr(W2), _ptr(y_perm), _ptr(ws),
                                  _nbytes(ws), _stream(stream)))


def moe_grouped_ffn(p, x_perm, offsets, W1, W2, y_perm, ws, stream=None):
    _check(load().moe_grouped_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(W1), _ptr(W2), _ptr(y_perm),
                                  _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_combine(p, y_perm, slot, topk_w, y, stream=None):
    _check(load().moe_combine(ctypes.byref(p), _ptr(y_perm), _ptr(slot), _ptr(topk_w), _ptr(y), _stream(stream)))


def moe_forward(p, x, Wg, bg, W1, W2, y, logits=None, info=None, ws=None, stream=None):
    """info: optional dict with any of topk_idx, topk_w, counts, offsets, slot, src_token tensors."""
    ri = None
    if info:
        ri = RouteInfo(*[_ptr(info.get(f)) for f, _ in RouteInfo._fields_])
    _check(load().moe_forward(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(y),
                              _ptr(logits), ctypes.byref(ri) if ri is not None else None, _ptr(ws), _nbytes(ws),
                              _stream(stream)))


def moe_forward_noalloc(p, x, Wg, bg, W1, W2, y, logits=None, info=None, stream=None):
    """moe_forward with the library's own device scratch as workspace (no
    allocation; problems up to 32 MiB of workspace)."""
    ri = None
    if info:
        ri = RouteInfo(*[_ptr(info.get(f)) for f, _ in RouteInfo._fields_])
    _check(load().moe_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(y),
                                      _ptr(logits), ctypes.byref(ri) if ri is not None else None, _stream(stream)))


def moe_router_stats(p, logits, counts, offsets, frac, mean_prob, scalars, ws, stream=None):
    """scalars [3] = (aux loss without coefficient, Z-loss, drop rate)."""
    _check(load().moe_router_stats(ctypes.byref(p), _ptr(logits), _ptr(counts), _ptr(offsets), _ptr(frac),
                                   _ptr(mean_prob), _ptr(scalars), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_shared_workspace_size(p, Fs) -> int:
    n = ctypes.c_size_t()
    _check(load().moe_shared_workspace_size(ctypes.byref(p), int(Fs), ctypes.byref(n)))
    return n.value


def moe_shared_expert(p, Fs, x, Ws1, Ws2, y_shared, ws, stream=None):
    _check(load().moe_shared_expert(ctypes.byref(p), int(Fs), _ptr(x), _ptr(Ws1), _ptr(Ws2), _ptr(y_shared),
                                    _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_combine_shared(p, y_perm, slot, topk_w, y_shared, y, stream=None):
    _check(load().moe_combine_shared(ctypes.byref(p), _ptr(y_perm), _ptr(slot), _ptr(topk_w), _ptr(y_shared),
                                     _ptr(y), _stream(stream)))


def moe_quantize_fp8(src, codes, scales, stream=None):
    """Rows of src (fp32 or bf16 tensor [rows, K]) to E4M3 codes (uint8 [rows, K])
    and power-of-two row scales (fp32 [rows])."""
    import torch
    dt = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}[src.dtype]
    rows, K = src.shape[0], src.numel() // max(src.shape[0], 1)
    _check(load().moe_quantize_fp8(_ptr(src), dt, rows, K, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_fp8_workspace_size(p) -> int:
    n = ctypes.c_size_t()
    _check(load().moe_fp8_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_expert_up_fp8(p, aq, a_scale, src_token, offsets, W1q, w1s, h, ws=None, stream=None):
    _check(load().moe_expert_up_fp8(ctypes.byref(p), _ptr(aq), _ptr(a_scale), _ptr(src_token), _ptr(offsets),
                                    _ptr(W1q), _ptr(w1s), _ptr(h), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_expert_down_fp8(p, hq, hs, offsets, W2q, w2s, y_perm, ws=None, stream=None):
    _check(load().moe_expert_down_fp8(ctypes.byref(p), _ptr(hq), _ptr(hs), _ptr(offsets), _ptr(W2q), _ptr(w2s),
                                      _ptr(y_perm), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_forward_fp8(p, x, Wg, bg, W1q, w1s, W2q, w2s, y, logits=None, info=None, ws=None, stream=None):
    ri = None
    if info:
        ri = RouteInfo(*[_ptr(info.get(f)) for f, _ in RouteInfo._fields_])
    _check(load().moe_forward_fp8(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1q), _ptr(w1s), _ptr(W2q),
                                  _ptr(w2s), _ptr(y), _ptr(logits), ctypes.byref(ri) if ri is not None else None,
                                  _ptr(ws), _nbytes(ws), _stream(stream)))


def _route_info(info):
    return RouteInfo(*[_ptr(info.get(f)) for f, _ in RouteInfo._fields_])


def _saved(saved):
    return Saved(*[_ptr(saved.get(f)) for f, _ in Saved._fields_])


def moe_forward_train(p, x, Wg, bg, W1, W2, y, logits, info, saved, ws=None, stream=None):
    """info: dict of every route-info tensor; saved: dict of u, h, y_perm tensors."""
    ri, sv = _route_info(info), _saved(saved)
    _check(load().moe_forward_train(ctypes.byref(p), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(y),
                                    _ptr(logits), ctypes.byref(ri), ctypes.byref(sv), _ptr(ws), _nbytes(ws),
                                    _stream(stream)))


def moe_backward_workspace_size(p) -> int:
    n = ctypes.c_size_t()
    _check(load().moe_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_backward(p, dy, x, Wg, W1, W2, logits, info, saved, dx, dWg, dbg, dW1, dW2, ws=None, stream=None,
                 aux_coef=0.0, z_coef=0.0):
    """aux_coef, z_coef: coefficients of the balancing losses (auxiliary
    loss, Z-loss) whose gradients are added; both 0 passes no losses."""
    ri = _route_info(info) if info is not None else None
    sv = _saved(saved) if saved is not None else None
    ls = RouterLosses(float(aux_coef), float(z_coef)) if (aux_coef or z_coef) else None
    _check(load().moe_backward(ctypes.byref(p), _ptr(dy), _ptr(x), _ptr(Wg), _ptr(W1), _ptr(W2), _ptr(logits),
                               ctypes.byref(ri) if ri is not None else None,
                               ctypes.byref(sv) if sv is not None else None,
                               ctypes.byref(ls) if ls is not None else None, _ptr(dx), _ptr(dWg), _ptr(dbg),
                               _ptr(dW1), _ptr(dW2), _ptr(ws), _nbytes(ws), _stream(stream)))
