"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Neighbour lists must match bit-exactly; attention outputs must be within
the tolerances of ``parity_util``.  The GPU side builds its own lists; the
oracle builds its own; inputs are the same seeded arrays.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from gen import make_case, stress_copy_rows, stress_duplicate_slots
from gen.synth import stress_rng
from parity_util import assert_finite, check_close, to_np, tol_for

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ca():
    import gathered_local_attention_amd as ca

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ca._lib.load()   # raises if the HIP library is missing
    return ca


def gpu_lists(ca, coords, G, k=6):
    perm, nbr, key_idx = ca.build_neighbors(torch.from_numpy(coords).to(DEV), G, k=k)
    torch.cuda.synchronize()
    return perm, nbr, key_idx


def assert_lists_equal(gpu, ref, what=""):
    for name, g, r in zip(("perm", "nbr", "key_idx"), gpu, ref):
        g = g.cpu().numpy()
        assert g.shape == r.shape, (name, g.shape, r.shape)
        diff = np.argwhere(g != r)
        assert diff.size == 0, f"{what} {name}: {len(diff)} mismatches, first at {diff[:3].tolist()}"


# ----------------------------------------------------------------------------
# neighbour lists
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,B", [("tiny", None), ("stage1", 32), ("stage3", 32), ("highres", 4)])
def test_neighbours_bit_exact(ca, name, B):
    case = make_case(name, B=B, tensors=False)
    cfg = case["cfg"]
    print(f"case {name} B={cfg.B} N={cfg.N}", flush=True)
    ref = O.build_neighbors(case["coords"], cfg.G)
    assert_lists_equal(gpu_lists(ca, case["coords"], cfg.G), ref, name)


def _jitter_coords(rng, G, B=1):
    cells = np.arange(G * G)
    xy = np.stack([cells % G, cells // G], 1) + rng.uniform(-0.5, 0.5, (G * G, 2))
    return np.repeat(xy[None].astype(np.float32), B, 0)


@pytest.mark.parametrize("G,k", [(72, 6), (48, 3), (40, 8), (16, 1)])
def test_neighbours_ragged_chunks_and_k(ca, G, k):
    """N = G*G not a multiple of the 2048-token sort chunk, several k."""
    rng = np.random.default_rng(G * 10 + k)
    coords = _jitter_coords(rng, G, B=2)
    coords[1] = coords[1][rng.permutation(G * G)]
    print(f"case jitter G={G} k={k}", flush=True)
    ref = O.build_neighbors(coords, G, k=k)
    assert_lists_equal(gpu_lists(ca, coords, G, k=k), ref, f"G={G}")


@pytest.mark.parametrize("N,k", [(9000, 6), (2056, 4)])
def test_neighbours_blobs_and_outliers(ca, N, k):
    """Uneven density (dense blobs of several widths, sparse background):
    the candidate search of large images skips tiles by their bounding
    boxes, and the lists must still be the exact ones."""
    rng = np.random.default_rng(N + k)
    G = 128
    centres = rng.uniform(0, G, (5, 2))
    widths = rng.uniform(0.3, 6.0, 5)
    lab = rng.integers(0, 5, N)
    xy = centres[lab] + rng.normal(0.0, 1.0, (N, 2)) * widths[lab, None]
    xy[: N // 50] = rng.uniform(0, G, (N // 50, 2))
    coords = np.stack([xy, xy[rng.permutation(N)]]).astype(np.float32)
    print(f"case blobs N={N} k={k}", flush=True)
    ref = O.build_neighbors(coords, G, k=k)
    assert_lists_equal(gpu_lists(ca, coords, G, k=k), ref, f"blobs N={N}")


def test_neighbours_with_code_ties_and_few_clusters(ca):
    rng = np.random.default_rng(3)
    # many tokens share a coordinate -> equal Morton codes, order by index
    pts = rng.integers(0, 6, size=(1, 4096, 2)).astype(np.float32)
    ref = O.build_neighbors(pts, 8)
    assert_lists_equal(gpu_lists(ca, pts, 8), ref, "ties")
    # fewer clusters than list entries -> -1 padding
    small = rng.uniform(0, 4, size=(3, 16, 2)).astype(np.float32)
    ref = O.build_neighbors(small, 4)
    assert_lists_equal(gpu_lists(ca, small, 4), ref, "small")
    # coordinates outside the grid clamp
    wild = rng.uniform(-20, 90, size=(2, 256, 2)).astype(np.float32)
    ref = O.build_neighbors(wild, 64)
    assert_lists_equal(gpu_lists(ca, wild, 64), ref, "clamp")


# ----------------------------------------------------------------------------
# forward / backward on small cases, every output compared
# ----------------------------------------------------------------------------

def run_case(ca, name, B=None, modify=None, check_bwd=True):
    case = make_case(name, B=B)
    cfg = case["cfg"]
    print(f"case {name} B={cfg.B} N={cfg.N} H={cfg.H} dtype={cfg.dtype}", flush=True)
    scale = 1.0 / math.sqrt(cfg.D)
    perm_g, _, key_g = gpu_lists(ca, case["coords"], cfg.G)
    perm_r, _, key_r = O.build_neighbors(case["coords"], cfg.G)
    assert np.array_equal(perm_g.cpu().numpy(), perm_r)
    assert np.array_equal(key_g.cpu().numpy(), key_r)
    if cfg.dup_frac:
        key_r = stress_duplicate_slots(key_r, cfg.cs, stress_rng(cfg), cfg.dup_frac)
        key_g = torch.from_numpy(stress_duplicate_slots(key_g.cpu().numpy(), cfg.cs,
                                                        stress_rng(cfg), cfg.dup_frac)).to(DEV)
        assert np.array_equal(key_g.cpu().numpy(), key_r)
    q, k, v, do = (case[n] for n in ("q", "k", "v", "do"))
    if modify is not None:
        q, k, v, do = modify(q, k, v, do)
    qi_r = perm_r.reshape(cfg.B, cfg.C, cfg.cs)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = ca.fwd(qd, kd, vd, perm_g, key_g, scale)
    torch.cuda.synchronize()
    tol = tol_for(cfg)
    o_r, lse_r = O.attn_fwd_gathered(q, k, v, qi_r, key_r, scale)
    assert_finite("O", o)
    assert_finite("LSE", lse)
    check_close("O", o, o_r, tol["o"], tol["rel"])
    check_close("LSE", lse, lse_r, tol["lse"], False)
    if not check_bwd:
        return
    dq, dk, dv = ca.bwd(qd, kd, vd, o, dod, lse, perm_g, key_g, scale)
    torch.cuda.synchronize()
    grads_r = O.attn_bwd_gathered(q, k, v, do, qi_r, key_r, scale)
    for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), grads_r):
        assert_finite(nm, g)
        check_close(nm, g, r, tol["g"], tol["rel"])
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, inputs=(qd, kd, vd, dod, perm_g, key_g, scale))


def test_tiny_fp32_forward(ca):
    run_case(ca, "tiny", check_bwd=False)


def test_tiny_fp32_backward(ca):
    run_case(ca, "tiny", check_bwd=True)


@pytest.mark.parametrize("name,B", [("stage1", 2), ("stage3", 3), ("stress", 2)])
def test_small_fwd_bwd(ca, name, B):
    run_case(ca, name, B=B)


def test_stress_equal_logits_reading(ca):
    """Second reading of the stress workload: copied K/V rows give exact
    logit ties across clusters."""
    def modify(q, k, v, do):
        k2, v2 = stress_copy_rows(k, v, np.random.default_rng(77), 0.1)
        return q, k2, v2, do
    run_case(ca, "stress", B=1, modify=modify)


def test_backward_is_deterministic(ca):
    r = run_case(ca, "stage1", B=2)
    qd, kd, vd, dod, perm, key, scale = r["inputs"]
    for _ in range(2):
        dq, dk, dv = ca.bwd(qd, kd, vd, r["o"], dod, r["lse"], perm, key, scale)
        torch.cuda.synchronize()
        assert torch.equal(dq, r["dq"]) and torch.equal(dk, r["dk"]) and torch.equal(dv, r["dv"])
    o, lse = ca.fwd(qd, kd, vd, perm, key, scale)
    assert torch.equal(o, r["o"]) and torch.equal(lse, r["lse"])


@pytest.mark.parametrize("scale", [0.2, -0.35, 0.0])
def test_holes_repeats_and_short_lists(ca, scale):
    """Hand-made lists: -1 slots, repeated slots, a cluster with a single
    valid slot, and k = 3 (24 slots), every dtype; a positive, a negative
    and a zero logit scale (the API takes any finite scale).  Random lists
    over all tokens pile many slots onto some keys, so |dV| reaches ~10
    where one bf16 output rounding step is 0.03: the bf16/f16 bars are
    taken relative to max(1, max|ref|)."""
    rng = np.random.default_rng(21)
    B, N, H, D = 2, 128, 3, 32
    for nk in (48, 24):
        for dt in (torch.float32, torch.bfloat16, torch.float16):
            print(f"case hand lists nk={nk} {dt} scale={scale}", flush=True)
            q_idx = np.stack([rng.permutation(N).reshape(-1, 8) for _ in range(B)]).astype(np.int32)
            key_idx = rng.integers(0, N, size=(B, N // 8, nk)).astype(np.int32)
            key_idx[:, :, 3] = key_idx[:, :, 2]
            key_idx[:, ::2, -1] = -1
            key_idx[:, 5, :] = -1
            key_idx[:, 5, 7] = 11
            q, k, v, do = (torch.randn(B, N, H, D, generator=torch.Generator().manual_seed(s)).to(dt)
                           for s in range(4))
            dev = [t.to(DEV) for t in (q, k, v, do)]
            qi, ki = torch.from_numpy(q_idx).to(DEV), torch.from_numpy(key_idx).to(DEV)
            o, lse = ca.fwd(dev[0], dev[1], dev[2], qi, ki, scale)
            dq, dk, dv = ca.bwd(dev[0], dev[1], dev[2], o, dev[3], lse, qi, ki, scale)
            torch.cuda.synchronize()
            o_r, lse_r = O.attn_fwd_dense(q, k, v, q_idx, key_idx, scale)
            g_r = O.attn_bwd_dense(q, k, v, do, q_idx, key_idx, scale)
            t = {torch.float32: (1e-5, 1e-5, 1e-5)}.get(dt, (1e-2, 1e-3, 2e-2))
            rel = dt != torch.float32
            check_close("O", o, o_r, t[0], rel)
            check_close("LSE", lse, lse_r, t[1], False)
            for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_r):
                check_close(nm, g, r, t[2], rel)


@pytest.mark.parametrize("N", [2304, 4608])
def test_grid_plan_random_lists(ca, N):
    """Images above the 2048-token in-LDS plan: 2304 tokens (288 clusters)
    take the 4096-token in-LDS plan (multiplicities accumulated in global
    memory), 4608 tokens the grid-wide transposition.  Random lists with -1
    slots, repeated slots and groups that mix clusters (the per-slot paths),
    plus build-style lists of whole clusters (the grouped paths)."""
    rng = np.random.default_rng(33)
    B, H, D, nk = 2, 2, 32, 48
    C = N // 8
    q_idx = np.stack([rng.permutation(N).reshape(-1, 8) for _ in range(B)]).astype(np.int32)
    key_rand = rng.integers(0, N, size=(B, C, nk)).astype(np.int32)
    key_rand[:, :, 5] = key_rand[:, :, 4]
    key_rand[:, ::3, -2:] = -1
    nb = (np.arange(C)[:, None] + np.array([0, 1, -1, 2, -2, 5])[None, :]) % C
    key_grp = np.stack([q_idx[b][nb].reshape(C, nk) for b in range(B)]).astype(np.int32)
    key_grp[:, 7] = key_rand[:, 7]   # one cluster with mixed groups in a grouped image
    for name, key_idx in (("random", key_rand), ("grouped", key_grp)):
        for dt in (torch.bfloat16, torch.float32):
            print(f"case plan N={N} {name} {dt}", flush=True)
            q, k, v, do = (torch.randn(B, N, H, D, generator=torch.Generator().manual_seed(40 + s)).to(dt)
                           for s in range(4))
            scale = 0.2
            dev = [t.to(DEV) for t in (q, k, v, do)]
            qi, ki = torch.from_numpy(q_idx).to(DEV), torch.from_numpy(key_idx).to(DEV)
            o, lse = ca.fwd(dev[0], dev[1], dev[2], qi, ki, scale)
            dq, dk, dv = ca.bwd(dev[0], dev[1], dev[2], o, dev[3], lse, qi, ki, scale)
            torch.cuda.synchronize()
            o_r, lse_r = O.attn_fwd_gathered(q, k, v, q_idx, key_idx, scale)
            g_r = O.attn_bwd_gathered(q, k, v, do, q_idx, key_idx, scale)
            t = {torch.float32: (1e-5, 1e-5, 1e-5)}.get(dt, (1e-2, 1e-3, 2e-2))
            rel = dt != torch.float32
            check_close("O", o, o_r, t[0], rel)
            check_close("LSE", lse, lse_r, t[1], False)
            for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_r):
                check_close(nm, g, r, t[2], rel)


def test_fully_masked_cluster(ca):
    B, N, H = 1, 64, 2
    q_idx = np.arange(N, dtype=np.int32).reshape(1, -1, 8)
    key_idx = np.tile(np.arange(48, dtype=np.int32), (1, N // 8, 1))
    key_idx[0, 2] = -1
    q, k, v = (torch.randn(B, N, H, 32) for _ in range(3))
    o, lse = ca.fwd(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(q_idx).to(DEV),
                    torch.from_numpy(key_idx).to(DEV), 0.2)
    torch.cuda.synchronize()
    rows = q_idx[0, 2]
    assert (o[0, rows] == 0).all()
    assert torch.isneginf(lse[0, rows]).all()
    o_r, _ = O.attn_fwd_dense(q, k, v, q_idx, key_idx, 0.2)
    check_close("O", o, o_r, 1e-5, False)


def test_empty_batch_is_noop(ca):
    q = torch.empty(0, 64, 2, 32, device=DEV, dtype=torch.bfloat16)
    qi = torch.empty(0, 8, 8, device=DEV, dtype=torch.int32)
    ki = torch.empty(0, 8, 48, device=DEV, dtype=torch.int32)
    o, lse = ca.fwd(q, q, q, qi, ki)
    assert o.shape == q.shape and lse.shape == (0, 64, 2)


def test_autograd_wrapper(ca):
    case = make_case("stage3", B=1)
    cfg = case["cfg"]
    perm, _, key = gpu_lists(ca, case["coords"], cfg.G)
    q, k, v = (case[n].to(DEV).requires_grad_(True) for n in ("q", "k", "v"))
    o = ca.cluster_attention(q, k, v, perm, key)
    o.backward(case["do"].to(DEV))
    o2, lse = ca.fwd(q.detach(), k.detach(), v.detach(), perm, key)
    g = ca.bwd(q.detach(), k.detach(), v.detach(), o2, case["do"].to(DEV), lse, perm, key)
    assert torch.equal(o.detach(), o2)
    for a, b in zip((q.grad, k.grad, v.grad), g):
        assert torch.equal(a, b)


# Whole-batch, every-element parity at the benchmarked launches lives in
# test_gpu_full_parity.py.


def test_planned_backward_equals_backward(ca):
    """The transposed lists built once (bwd_plan) and reused: bit-identical
    to the self-planning backward, on the in-LDS plan (stage-1 images), the
    grid-wide plan (a packed batch) and the vector-ALU kernels (fp32), and
    across two calls with different output gradients."""
    from gen import make_varlen_case

    r = run_case(ca, "stage1", B=2)
    qd, kd, vd, dod, perm, key, scale = r["inputs"]
    plan = ca.bwd_plan(perm, key, qd.shape[1])
    for do in (dod, dod.flip(1).contiguous()):
        ref = ca.bwd(qd, kd, vd, r["o"], do, r["lse"], perm, key, scale)
        got = ca.bwd(qd, kd, vd, r["o"], do, r["lse"], perm, key, scale, plan=plan)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    for name in ("varlen_mixed", "varlen_tiny", "varlen"):
        case = make_varlen_case(name)
        print(f"case planned {name}", flush=True)
        q_idx, _, key_v, _, _ = ca.build_neighbors_varlen(torch.from_numpy(case["coords"]).to(DEV),
                                                          case["lengths"], case["cfg"].G)
        dev = [case[n].to(DEV) for n in ("q", "k", "v", "do")]
        o, lse = ca.fwd_varlen(dev[0], dev[1], dev[2], q_idx, key_v)
        plan = ca.bwd_plan(q_idx, key_v, dev[0].shape[0])
        plan_img = ca.bwd_plan_varlen(q_idx, key_v, case["lengths"])   # one workgroup per image
        ref = ca.bwd_varlen(dev[0], dev[1], dev[2], o, dev[3], lse, q_idx, key_v)
        for p in (plan, plan_img):
            got = ca.bwd_varlen(dev[0], dev[1], dev[2], o, dev[3], lse, q_idx, key_v, plan=p)
            torch.cuda.synchronize()
            for a, b in zip(ref, got):
                assert torch.equal(a, b)
