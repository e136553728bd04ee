"""The allocation-free forward (moe_forward_noalloc), through the C ABI,
against moe_forward on the same inputs: two calls in a row, the second on a
smaller batch, each compared with moe_forward.  Routing, counts, offsets,
slots and source tokens must be identical (same kernels); y within the bf16
bar max|a - b| / max|b| <= 2e-2 (the allocation-free forward runs the grouped
GEMMs without the K split of their last round, another fp32 summation order).
The Mixtral widths (d = 4096, F = 14336, 8 experts, top-2, SwiGLU) at 256 and
then 37 tokens fit the 32 MiB scratch."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_logit_amd as moe
from _gpu import TOL, host, maxrel, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

T0, D, E, K, F = 256, 4096, 8, 2, 14336


def buffers(T):
    return {"topk_idx": torch.empty(T, K, dtype=torch.int32, device="cuda"),
            "topk_w": torch.empty(T, K, dtype=torch.float32, device="cuda"),
            "counts": torch.empty(E, dtype=torch.int32, device="cuda"),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device="cuda"),
            "slot": torch.empty(T, K, dtype=torch.int32, device="cuda"),
            "src_token": torch.empty(T * K, dtype=torch.int32, device="cuda")}


def test_noalloc_forward_matches_forward_twice():
    g = torch.Generator(device="cuda")
    g.manual_seed(20261203)
    bf = torch.bfloat16
    W1 = (torch.randn(E, 2 * F, D, generator=g, device="cuda") * 0.02).to(bf)
    W2 = (torch.randn(E, D, F, generator=g, device="cuda") * 0.02).to(bf)
    Wg = (torch.randn(E, D, generator=g, device="cuda") * 0.02).to(bf)
    bg = torch.linspace(0.5, -0.5, E, device="cuda")
    x_all = torch.randn(T0, D, generator=g, device="cuda").to(bf)
    for T in (T0, 37):
        print(f"[noalloc] T={T} d={D} E={E} k={K} F={F} swiglu bf16", flush=True)
        p = moe.problem(T, D, E, K, F, act="swiglu", dtype="bf16")
        x = x_all[:T].contiguous()
        ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
        ref_info, got_info = buffers(T), buffers(T)
        ref_y = torch.empty(T, D, dtype=bf, device="cuda")
        got_y = torch.full((T, D), float("nan"), dtype=bf, device="cuda")
        ref_z = torch.empty(T, E, dtype=torch.float32, device="cuda")
        got_z = torch.empty(T, E, dtype=torch.float32, device="cuda")
        moe.moe_forward(p, x, Wg, bg, W1, W2, ref_y, logits=ref_z, info=ref_info, ws=ws)
        moe.moe_forward_noalloc(p, x, Wg, bg, W1, W2, got_y, logits=got_z, info=got_info)
        torch.cuda.synchronize()
        assert np.array_equal(host(got_z), host(ref_z))
        for key in ref_info:
            a, b = host(got_info[key]), host(ref_info[key])
            if key == "src_token":
                P = int(host(ref_info["offsets"])[-1])
                a, b = a[:P], b[:P]
            assert np.array_equal(a, b), key
        err = maxrel(host(got_y), to_f64(host(ref_y)))
        print(f"  max-abs-rel vs moe_forward {err:.2e}", flush=True)
        assert err <= TOL["bf16"]
        del ws


def test_noalloc_forward_rejects_oversize_problem():
    p = moe.problem(4096, D, E, K, F, act="swiglu", dtype="bf16")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(p, torch.empty(1, device="cuda"), torch.empty(1, device="cuda"), None,
                                torch.empty(1, device="cuda"), torch.empty(1, device="cuda"),
                                torch.empty(1, device="cuda"))
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
