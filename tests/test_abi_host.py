"""C-ABI host checks: the library loads, exports every declared entry point,
sizes workspaces and capacities, and rejects bad arguments before anything is
enqueued.  No kernel is launched (these run without a GPU)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_logit_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = moe.load()
    names = declared_entry_points()
    assert set(names) >= {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTS)


def test_status_strings():
    lib = moe.load()
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE"


# The last rows use factors that are not exact in fp32 at shapes where the
# decimal factor times T*k/E is an integer: both sides take the fp32 value.
@pytest.mark.parametrize("T,E,k,cf", [(4096, 16, 2, 1.25), (10, 3, 1, 1.0), (8, 4, 2, 1e-30), (4096, 8, 2, 0.0),
                                      (4096, 8, 2, -1.0), (16384, 512, 2, 0.25), (1, 1, 1, 3.0),
                                      (100, 1, 1, 0.1), (100, 1, 1, 0.3), (100, 1, 1, 0.7), (100, 1, 1, 1.1),
                                      (1000, 10, 1, 0.3), (10, 1, 1, 0.3), (1000, 4, 2, 0.3), (600, 8, 2, 0.7),
                                      (1 << 24, 1024, 8, 0.1)])
def test_capacity_matches_oracle(T, E, k, cf):
    p = moe.problem(T, 64, E, k, 64, cf=cf)
    assert moe.moe_capacity(p) == oracle.capacity(T, E, k, cf)


def partial_floats(T, E, k, b, cf):
    """One partial output tile of the grouped GEMM's K-split last round, by
    the tile shape the expected rows per expert select."""
    rows = T * k // E
    C = oracle.capacity(T, E, k, cf)
    if C >= 0:
        rows = min(rows, C)
    if b == 4:
        return 128 * 128
    # from 256 rows on the bf16 forward may take the 256 x 256 tile (where K
    # is long enough), so the workspace holds partial tiles of that size
    return 256 * 256 if rows >= 256 else 128 * 128 if rows >= 128 else 64 * 256


def workspace_formula(T, d, E, k, F, b, cf=0.0):
    r = lambda n: (n + 255) // 256 * 256
    nch = max((T + 255) // 256, 1)
    gather = T * d * b < 0xF0000000  # else x_perm is kept in the workspace
    nstat = max((T + 3) // 4 if T < 1024 else 256, 1)  # blocks of the router statistics' first pass
    return (r(T * k * 4) * 4 + r(E * 4) + r((E + 1) * 4) + r(nch * E * 4) + r(T * E * 4)
            + r((nstat + 1) * (E + 1) * 8)
            + r(256 * partial_floats(T, E, k, b, cf) * 4) + r(T * k * F * b) + r(T * k * d * b)
            + (0 if gather else r(T * k * d * b)))


@pytest.mark.parametrize("T,d,E,k,F,dt,cf", [(256, 64, 4, 2, 128, "f32", 0.0),
                                             (4096, 4096, 8, 2, 14336, "bf16", 0.0),
                                             (1, 64, 1, 1, 64, "bf16", 0.0),
                                             (8192, 512, 64, 2, 1024, "bf16", 0.0),
                                             (16384, 1024, 512, 2, 512, "bf16", 0.0),
                                             (8192, 2048, 16, 2, 1408, "bf16", 1.25),
                                             (8192, 2048, 64, 2, 1408, "bf16", 0.25),
                                             (1 << 21, 2048, 64, 2, 1024, "bf16", 0.0)])
def test_workspace_size(T, d, E, k, F, dt, cf):
    p = moe.problem(T, d, E, k, F, dtype=dt, cf=cf)
    assert moe.moe_workspace_size(p) == workspace_formula(T, d, E, k, F, 4 if dt == "f32" else 2, cf)


BAD = [
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(E=0), moe.MOE_ERR_INVALID_ARG),
    (dict(E=1025), moe.MOE_ERR_UNSUPPORTED),
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=9, E=16), moe.MOE_ERR_UNSUPPORTED),
    (dict(k=5, E=4), moe.MOE_ERR_INVALID_ARG),
    (dict(d=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(F=32), moe.MOE_ERR_UNSUPPORTED),
    (dict(act=7), moe.MOE_ERR_INVALID_ARG),
    (dict(dtype=5), moe.MOE_ERR_INVALID_ARG),
    (dict(normalize=True, lam=0.0), moe.MOE_ERR_INVALID_ARG),
    (dict(normalize=True, lam=float("inf")), moe.MOE_ERR_INVALID_ARG),
    (dict(cf=float("nan")), moe.MOE_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", BAD)
def test_bad_problem_rejected(kw, status):
    args = dict(T=64, d=64, E=8, k=2, F=64)
    args.update(kw)
    p = moe.problem(args.pop("T"), args.pop("d"), args.pop("E"), args.pop("k"), args.pop("F"), **args)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(p)
    assert ei.value.status == status
    assert moe.load().moe_last_error()


FAKE = 1 << 20  # a 16-byte aligned, never dereferenced address


def test_bad_pointers_rejected_before_launch():
    p = moe.problem(64, 64, 8, 2, 64)
    ws = moe.moe_workspace_size(p)
    lib = moe.load()
    pp = ctypes.byref(p)
    # x given without Wg
    assert lib.moe_route(pp, FAKE, None, None, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # missing logits
    assert lib.moe_route(pp, None, None, None, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # misaligned x
    assert lib.moe_route(pp, FAKE + 2, FAKE, None, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert b"aligned" in lib.moe_last_error()
    # workspace too small
    assert lib.moe_permute(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_grouped_ffn(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == moe.MOE_ERR_WORKSPACE
    # forward without Wg and without logits
    assert lib.moe_forward(pp, FAKE, None, None, FAKE, FAKE, FAKE, None, None, FAKE, ws, None) == \
        moe.MOE_ERR_INVALID_ARG
    # null outputs
    assert lib.moe_combine(pp, FAKE, FAKE, FAKE, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_up(pp, FAKE, None, FAKE, FAKE, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down(pp, FAKE, FAKE, None, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    # a workspace, when given, must be large enough
    assert lib.moe_expert_up(pp, FAKE, None, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_expert_down(pp, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == moe.MOE_ERR_WORKSPACE
    # misaligned gather index
    assert lib.moe_expert_up(pp, FAKE, FAKE + 1, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG


def test_gather_limited_to_32_bit_offsets():
    # x of 8 GiB cannot be read through src_token; x_perm must be passed
    p = moe.problem(1 << 21, 2048, 64, 2, 1024)
    lib = moe.load()
    pp = ctypes.byref(p)
    assert lib.moe_expert_up(pp, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_UNSUPPORTED
    assert b"gather" in lib.moe_last_error()


def test_empty_problem_is_a_no_op():
    p = moe.problem(0, 64, 8, 2, 64)
    lib = moe.load()
    pp = ctypes.byref(p)
    # T == 0: nothing to do, no pointer is touched
    assert lib.moe_forward(pp, None, None, None, None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert lib.moe_route(pp, None, None, None, None, None, None, None) == moe.MOE_OK


@pytest.mark.parametrize("T,d,F,Fs,dt", [(4096, 4096, 14336, 1408, "bf16"), (100, 64, 64, 128, "f32"),
                                         (600, 256, 448, 2048, "bf16")])
def test_shared_workspace_size(T, d, F, Fs, dt):
    p = moe.problem(T, d, 8, 2, F, dtype=dt)
    b = 4 if dt == "f32" else 2
    r = lambda n: (n + 255) // 256 * 256
    # hidden rows [T][Fs], then the K-split partial tiles of a T-row segment
    tile = 128 * 128 if b == 4 else 256 * 256 if T >= 512 else 128 * 128 if T >= 128 else 64 * 256
    assert moe.moe_shared_workspace_size(p, Fs) == r(T * Fs * b) + r(256 * tile * 4)


def test_new_entry_points_reject_bad_arguments():
    p = moe.problem(64, 64, 8, 2, 64)
    ws = moe.moe_workspace_size(p)
    lib = moe.load()
    pp = ctypes.byref(p)
    # statistics: null output, short workspace
    assert lib.moe_router_stats(pp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_router_stats(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == moe.MOE_ERR_WORKSPACE
    # shared expert: bad hidden width, short workspace, null weights
    for Fs in (0, 96, 1 << 17):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_shared_workspace_size(p, Fs)
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    sws = moe.moe_shared_workspace_size(p, 128)
    assert lib.moe_shared_expert(pp, 128, FAKE, FAKE, FAKE, FAKE, FAKE, sws - 1, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_shared_expert(pp, 128, FAKE, None, FAKE, FAKE, FAKE, sws, None) == moe.MOE_ERR_INVALID_ARG
    # combine with a shared output: misaligned y_shared
    assert lib.moe_combine_shared(pp, FAKE, FAKE, FAKE, FAKE + 4, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op for all of them
    p0 = moe.problem(0, 64, 8, 2, 64)
    p0p = ctypes.byref(p0)
    assert lib.moe_router_stats(p0p, None, None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert lib.moe_shared_expert(p0p, 128, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert lib.moe_combine_shared(p0p, None, None, None, None, None, None) == moe.MOE_OK


def test_fp8_entry_points_reject_bad_arguments():
    lib = moe.load()
    # activations must be bf16, d and F multiples of 128
    for kw in (dict(dtype="f32"), dict(d=192), dict(F=320)):
        a = dict(T=64, d=256, E=8, k=2, F=256)
        a.update(kw)
        p = moe.problem(a.pop("T"), a.pop("d"), a.pop("E"), a.pop("k"), a.pop("F"), **a)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_fp8_workspace_size(p)
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    p = moe.problem(64, 256, 8, 2, 256)
    pp = ctypes.byref(p)
    ws = moe.moe_fp8_workspace_size(p)
    assert ws > moe.moe_workspace_size(p)
    r = lambda n: (n + 255) // 256 * 256
    assert ws == moe.moe_workspace_size(p) + r(64 * 256) + r(64 * 4) + r(128 * 256) + r(128 * 4)
    # quantiser: bad dtype, bad K, misaligned codes; zero rows is a no-op
    assert lib.moe_quantize_fp8(FAKE, 7, 4, 64, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(FAKE, moe.MOE_BF16, 4, 96, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_fp8(FAKE, moe.MOE_BF16, 4, 64, FAKE + 4, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(None, moe.MOE_BF16, 0, 64, None, None, None) == moe.MOE_OK
    # forward: short workspace; up/down: null scales
    assert lib.moe_forward_fp8(pp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws - 1,
                               None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_expert_up_fp8(pp, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down_fp8(pp, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG


def test_fp8_gather_limited_to_32_bit_offsets():
    # 2^20 tokens x 4096 codes = 4 GiB: the token codes cannot be gathered
    # through src_token (32-bit byte offsets); the limit is T*d < 0xF0000000
    lib = moe.load()
    big = moe.problem(1 << 20, 4096, 8, 2, 256)
    pb = ctypes.byref(big)
    assert lib.moe_expert_up_fp8(pb, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == \
        moe.MOE_ERR_UNSUPPORTED
    assert b"gather" in lib.moe_last_error()
    ws = moe.moe_fp8_workspace_size(big)
    assert lib.moe_forward_fp8(pb, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws,
                               None) == moe.MOE_ERR_UNSUPPORTED
    # without src_token the codes are permuted rows, addressed per tile: accepted past validation
    # (the workspace check is the next one to fail here)
    assert lib.moe_expert_up_fp8(pb, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == \
        moe.MOE_ERR_WORKSPACE
    # just below the limit the gather is accepted
    ok = moe.problem(983040 - 1, 4096, 8, 2, 256)   # (983040 - 1) * 4096 < 0xF0000000
    po = ctypes.byref(ok)
    assert lib.moe_expert_up_fp8(po, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == \
        moe.MOE_ERR_WORKSPACE


def backward_formula(T, d, E, k, F, act, b):
    r = lambda n: (n + 255) // 256 * 256
    n1 = 2 * F if act == "swiglu" else F
    ld = (T * k + 64 * E + 63) // 64 * 64
    nch = max((T + 63) // 64, 1)  # token chunks of the gate gradients' first pass
    tile = 128 * 128 if b == 4 else 256 * 256 if T * k // E >= 512 else 128 * 128 if T * k // E >= 128 else 64 * 256
    return (r(T * k * d * b) + r(T * k * 4) + r(T * E * 4) + r(T * k * n1 * b) + r(T * k * d * b)
            + (r(E * n1 * d * b) + r(E * d * F * b) if b == 4 else 0)  # transposed weights, fp32 only
            + r((E + 1) * 4)
            + r(d * ld * b) + r(F * ld * b) + r(n1 * ld * b) + r(d * ld * b)
            + r(nch * E * (d + 1) * 4) + r(256 * tile * 4))


@pytest.mark.parametrize("T,d,E,k,F,act,dt", [(4096, 4096, 8, 2, 14336, "swiglu", "bf16"),
                                              (256, 64, 4, 2, 128, "relu", "f32"),
                                              (16384, 1024, 512, 2, 512, "relu", "bf16"),
                                              (1, 64, 1, 1, 64, "swiglu", "bf16")])
def test_backward_workspace_size(T, d, E, k, F, act, dt):
    p = moe.problem(T, d, E, k, F, act=act, dtype=dt)
    b = 4 if dt == "f32" else 2
    assert moe.moe_backward_workspace_size(p) == backward_formula(T, d, E, k, F, act, b)


def test_backward_entry_points_reject_bad_arguments():
    lib = moe.load()
    # transposed row operands beyond 32-bit offsets
    big = moe.problem(1 << 21, 2048, 64, 2, 1024)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_backward_workspace_size(big)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    p = moe.problem(64, 64, 8, 2, 64)
    pp = ctypes.byref(p)
    bws = moe.moe_backward_workspace_size(p)
    ws = moe.moe_workspace_size(p)
    info = moe.RouteInfo(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    saved = moe.Saved(FAKE, FAKE, FAKE)
    ri, sv = ctypes.byref(info), ctypes.byref(saved)
    # the training forward needs info and saved, and a full workspace
    assert lib.moe_forward_train(pp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, ri, None, FAKE, ws, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_train(pp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, ri, sv, FAKE, ws - 1, None) == \
        moe.MOE_ERR_WORKSPACE
    bad_saved = moe.Saved(FAKE, FAKE + 2, FAKE)
    assert lib.moe_forward_train(pp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, ri, ctypes.byref(bad_saved), FAKE,
                                 ws, None) == moe.MOE_ERR_INVALID_ARG
    # dy, x, Wg, W1, W2, logits, info, saved, losses, dx, dWg, dbg, dW1, dW2, ws, ws_bytes, stream
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ri, sv, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bws, None]
    # short workspace; no route info; a gate without its gradient outputs; null dW2
    a = list(args)
    a[-2] = bws - 1
    assert lib.moe_backward(pp, *a) == moe.MOE_ERR_WORKSPACE
    a = list(args)
    a[6] = None
    assert lib.moe_backward(pp, *a) == moe.MOE_ERR_INVALID_ARG
    a = list(args)
    a[10] = None
    assert lib.moe_backward(pp, *a) == moe.MOE_ERR_INVALID_ARG
    a = list(args)
    a[13] = None
    assert lib.moe_backward(pp, *a) == moe.MOE_ERR_INVALID_ARG
    # balancing losses: non-finite coefficients; the auxiliary loss needs the counts
    for bad in (moe.RouterLosses(float("nan"), 0.0), moe.RouterLosses(0.0, float("inf"))):
        a = list(args)
        a[8] = ctypes.byref(bad)
        assert lib.moe_backward(pp, *a) == moe.MOE_ERR_INVALID_ARG
    no_counts = moe.RouteInfo(FAKE, FAKE, None, FAKE, FAKE, FAKE)
    aux = moe.RouterLosses(0.01, 0.0)
    a = list(args)
    a[6], a[8] = ctypes.byref(no_counts), ctypes.byref(aux)
    assert lib.moe_backward(pp, *a) == moe.MOE_ERR_INVALID_ARG
    assert b"counts" in lib.moe_last_error()
    # T == 0: the training forward is a no-op; the backward still needs its weight-gradient outputs
    p0 = moe.problem(0, 64, 8, 2, 64)
    p0p = ctypes.byref(p0)
    assert lib.moe_forward_train(p0p, None, None, None, None, None, None, None, None, None, None, 0, None) == \
        moe.MOE_OK
    assert lib.moe_backward(p0p, None, None, None, None, None, None, None, None, None, None, None, None, None, None,
                            None, 0, None) == moe.MOE_ERR_INVALID_ARG


def test_noalloc_forward_rejects_before_any_device_call():
    lib = moe.load()
    # the Mixtral-shaped layer needs ~235 MB of workspace: beyond the 32 MiB scratch
    big = moe.problem(4096, 4096, 8, 2, 14336, act="swiglu")
    pb = ctypes.byref(big)
    assert lib.moe_forward_noalloc(pb, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None) == \
        moe.MOE_ERR_WORKSPACE
    assert b"scratch" in lib.moe_last_error()
    small = moe.problem(64, 64, 8, 2, 64)
    ps = ctypes.byref(small)
    # bad pointers and missing logits are rejected as in moe_forward
    assert lib.moe_forward_noalloc(ps, FAKE, FAKE, None, FAKE, FAKE, None, None, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_noalloc(ps, FAKE, None, None, FAKE, FAKE, FAKE, None, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op
    p0 = moe.problem(0, 64, 8, 2, 64)
    assert lib.moe_forward_noalloc(ctypes.byref(p0), None, None, None, None, None, None, None, None, None) == \
        moe.MOE_OK
