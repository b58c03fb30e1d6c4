"""The backward that allocates nothing (cluster_attn_bwd_planned_noalloc).

Called through the C-ABI (ctypes, device pointers) on the same inputs as
cluster_attn_bwd_planned, two calls in a row with the second one smaller
(the library's scratch still holds the first call's pairs): dQ, dK and dV
must equal the workspace entry point's bit for bit (same kernels, same
arithmetic).  Sizes beyond the scratch are refused on the host before any
launch.
"""

import ctypes
import math

import pytest
import torch

from gen import make_case

DEV = "cuda:0"


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.gpu
def test_noalloc_backward_equals_planned_backward():
    import gathered_local_attention_amd as ca

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib = ca._lib.load()
    for B in (8, 3):   # the second call is smaller
        case = make_case("stage1", B=B)
        cfg = case["cfg"]
        print(f"case stage1 B={B} noalloc backward", flush=True)
        scale = 1.0 / math.sqrt(cfg.D)
        perm, _, key = ca.build_neighbors(torch.from_numpy(case["coords"]).to(DEV), cfg.G)
        q, k, v, do = (case[n].to(DEV) for n in ("q", "k", "v", "do"))
        o, lse = ca.fwd(q, k, v, perm, key, scale)
        plan = ca.bwd_plan(perm, key, cfg.N)
        ref = ca.bwd(q, k, v, o, do, lse, perm, key, scale, plan=plan)
        out = [torch.full_like(q, float("nan")) for _ in range(3)]
        C, nk = key.shape[1], key.shape[2]
        rc = lib.cluster_attn_bwd_planned_noalloc(
            1, cfg.B, cfg.N, C, cfg.H, cfg.D, 8, nk, ctypes.c_float(scale), _ptr(q), _ptr(k),
            _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(perm), _ptr(key), _ptr(plan),
            ctypes.c_size_t(plan.numel()), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, lib.cluster_attn_last_error().decode()
        torch.cuda.synchronize()
        for nm, a, r in zip(("dQ", "dK", "dV"), out, ref):
            assert torch.equal(a, r), f"{nm} differs from cluster_attn_bwd_planned (B={B})"
        got = ca.bwd_planned_noalloc(q, k, v, o, do, lse, perm, key, plan, scale)
        torch.cuda.synchronize()
        for nm, a, r in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, r), f"{nm} (binding) differs (B={B})"


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """Host-side check, no device pointer is touched (none is valid here)."""
    import gathered_local_attention_amd as ca

    lib = ca._lib.load()
    rows = lib.cluster_attn_bwd_planned_noalloc_max_rows()
    assert rows == ((32 << 20) - 256) // 8
    fake = ctypes.c_void_p(16)
    N, H = 1 << 20, 8                 # 8,388,608 rows of pairs
    args = [1, 1, N, N // 8, H, 32, 8, 48, ctypes.c_float(0.1)] + [fake] * 9 + \
           [ctypes.c_size_t(1 << 40)] + [fake] * 3 + [ctypes.c_void_p(0)]
    rc = lib.cluster_attn_bwd_planned_noalloc(*args)
    assert rc != 0
    assert "scratch" in lib.cluster_attn_last_error().decode()
