"""GPU parity of ragged geometry against the fp64 oracle, through the C ABI:
images whose token count is not a multiple of 8 (a partial last cluster)
and packed batches of images of different sizes.  Lists bit-exact; outputs
within the tolerances of ``parity_util``."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from gen import RaggedConfig, make_case, make_varlen_case
from parity_util import assert_finite, check_close, tol_for, TOL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ca():
    import gathered_local_attention_amd as ca

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ca._lib.load()
    return ca


def _equal(name, got, ref):
    g = got.cpu().numpy()
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    diff = np.argwhere(g != ref)
    assert diff.size == 0, f"{name}: {len(diff)} mismatches, first at {diff[:3].tolist()}"


# ----------------------------------------------------------------------------
# lists
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["stage2", "stage4"])
def test_partial_cluster_lists_bit_exact(ca, name):
    case = make_case(name, tensors=False)
    cfg = case["cfg"]
    print(f"case {name} B={cfg.B} N={cfg.N}", flush=True)
    got = ca.build_neighbors(torch.from_numpy(case["coords"]).to(DEV), cfg.G)
    ref = O.build_neighbors(case["coords"], cfg.G)
    for nm, g, r in zip(("perm", "nbr", "key_idx"), got, ref):
        _equal(nm, g, r)


@pytest.mark.parametrize("N,k", [(4100, 6), (2049, 3), (6001, 8), (1, 6), (13, 2)])
def test_partial_cluster_lists_large_and_small(ca, N, k):
    """Images above the in-LDS limit (segment / merge path) and tiny ones,
    every remainder class of N mod 8 among them."""
    rng = np.random.default_rng(N + k)
    G = 128
    coords = rng.uniform(-0.5, G - 0.5, size=(2, N, 2)).astype(np.float32)
    coords[1, N // 2:] = coords[1, : N - N // 2]                # repeated points: ties
    print(f"case ragged N={N} k={k}", flush=True)
    got = ca.build_neighbors(torch.from_numpy(coords).to(DEV), G, k=k)
    ref = O.build_neighbors(coords, G, k=k)
    for nm, g, r in zip(("perm", "nbr", "key_idx"), got, ref):
        _equal(nm, g, r)


def _varlen_lists(ca, case, k=6):
    cfg = case["cfg"]
    got = ca.build_neighbors_varlen(torch.from_numpy(case["coords"]).to(DEV), case["lengths"],
                                    cfg.G, k=k)
    ref = O.build_neighbors_varlen(case["coords"], case["lengths"], cfg.G, k=k)
    for nm, g, r in zip(("q_idx", "nbr", "key_idx", "tok_off", "clu_off"), got, ref):
        _equal(nm, g, r.astype(np.int32))
    return got, ref


@pytest.mark.parametrize("name", ["varlen_tiny", "varlen_mixed", "varlen"])
def test_varlen_lists_bit_exact(ca, name):
    case = make_varlen_case(name, tensors=False)
    print(f"case {name} lengths {case['lengths'][:8]}...", flush=True)
    _varlen_lists(ca, case)


def test_varlen_edge_batches(ca):
    """All images empty but one; a single image; k = 1."""
    rng = np.random.default_rng(5)
    for lengths, k in (((0, 0, 7, 0), 6), ((3000,), 4), ((9, 1, 16), 1)):
        T = sum(lengths)
        coords = rng.uniform(0, 63, size=(T, 2)).astype(np.float32)
        print(f"case varlen edges {lengths} k={k}", flush=True)
        cfg = RaggedConfig("edge", 0, len(lengths), 64, 1, 32, "f32", "cells", lengths)
        _varlen_lists(ca, {"cfg": cfg, "coords": coords, "lengths": list(lengths)}, k=k)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def _check_all(o, lse, grads, ref_o, ref_lse, ref_g, tol):
    for nm, t in (("O", o), ("LSE", lse)) + tuple(zip(("dQ", "dK", "dV"), grads)):
        assert_finite(nm, t)
    check_close("O", o, ref_o, tol["o"], tol["rel"])
    check_close("LSE", lse, ref_lse, tol["lse"], False)
    for nm, g, r in zip(("dQ", "dK", "dV"), grads, ref_g):
        check_close(nm, g, r, tol["g"], tol["rel"])


@pytest.mark.parametrize("name,B", [("stage4", 2), ("stage2", 2)])
def test_partial_cluster_attention(ca, name, B):
    case = make_case(name, B=B)
    cfg = case["cfg"]
    print(f"case {name} B={B} N={cfg.N} H={cfg.H}", flush=True)
    scale = 1.0 / math.sqrt(cfg.D)
    perm, _, key = ca.build_neighbors(torch.from_numpy(case["coords"]).to(DEV), cfg.G)
    perm_r, _, key_r = O.build_neighbors(case["coords"], cfg.G)
    qi_r = perm_r.reshape(B, cfg.C, 8)
    dev = [case[n].to(DEV) for n in ("q", "k", "v", "do")]
    o, lse = ca.fwd(dev[0], dev[1], dev[2], perm, key, scale)
    g = ca.bwd(dev[0], dev[1], dev[2], o, dev[3], lse, perm, key, scale)
    torch.cuda.synchronize()
    o_r, lse_r = O.attn_fwd_gathered(case["q"], case["k"], case["v"], qi_r, key_r, scale)
    g_r = O.attn_bwd_gathered(case["q"], case["k"], case["v"], case["do"], qi_r, key_r, scale)
    _check_all(o, lse, g, o_r, lse_r, g_r, tol_for(cfg))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_partial_cluster_attention_every_remainder(ca, dt):
    """N = 8m + r for r = 1..7 (fp32: vector-ALU kernels; bf16: matrix-core
    kernels), odd head count."""
    rng = np.random.default_rng(17)
    for r in range(1, 8):
        N, H = 40 + r, 3
        coords = rng.uniform(0, 15, size=(2, N, 2)).astype(np.float32)
        q, k, v, do = (torch.randn(2, N, H, 32, generator=torch.Generator().manual_seed(10 * r + s)).to(dt)
                       for s in range(4))
        print(f"case remainder r={r} {dt}", flush=True)
        perm, _, key = ca.build_neighbors(torch.from_numpy(coords).to(DEV), 16)
        perm_r, _, key_r = O.build_neighbors(coords, 16)
        _equal("perm", perm, perm_r)
        dev = [t.to(DEV) for t in (q, k, v, do)]
        o, lse = ca.fwd(dev[0], dev[1], dev[2], perm, key, 0.2)
        g = ca.bwd(dev[0], dev[1], dev[2], o, dev[3], lse, perm, key, 0.2)
        torch.cuda.synchronize()
        qi_r = perm_r.reshape(2, -1, 8)
        o_r, lse_r = O.attn_fwd_dense(q, k, v, qi_r, key_r, 0.2)
        g_r = O.attn_bwd_dense(q, k, v, do, qi_r, key_r, 0.2)
        _check_all(o, lse, g, o_r, lse_r, g_r, TOL["f32" if dt == torch.float32 else "bf16"])


@pytest.mark.parametrize("name", ["varlen_tiny", "varlen_mixed"])
def test_varlen_attention(ca, name):
    case = make_varlen_case(name)
    cfg = case["cfg"]
    print(f"case {name} T={case['coords'].shape[0]} H={cfg.H} {cfg.dtype}", flush=True)
    scale = 1.0 / math.sqrt(cfg.D)
    (q_idx, _, key, _, _), (qi_r, _, key_r, _, _) = _varlen_lists(ca, case)
    dev = [case[n].to(DEV) for n in ("q", "k", "v", "do")]
    o, lse = ca.fwd_varlen(dev[0], dev[1], dev[2], q_idx, key, scale)
    g = ca.bwd_varlen(dev[0], dev[1], dev[2], o, dev[3], lse, q_idx, key, scale)
    torch.cuda.synchronize()
    one = lambda n: case[n][None]
    o_r, lse_r = O.attn_fwd_gathered(one("q"), one("k"), one("v"), qi_r[None], key_r[None], scale)
    g_r = O.attn_bwd_gathered(one("q"), one("k"), one("v"), one("do"), qi_r[None], key_r[None], scale)
    _check_all(o[None], lse[None], [t[None] for t in g], o_r, lse_r, g_r, TOL[cfg.dtype])


def test_varlen_full_batch_every_element(ca):
    """The 32-image packed batch as the benchmark runs it (lists, a plan
    built one workgroup per image, forward and planned backward): every
    element against the oracle."""
    case = make_varlen_case("varlen")
    cfg = case["cfg"]
    T = case["coords"].shape[0]
    print(f"case varlen full T={T} (every element)", flush=True)
    scale = 1.0 / math.sqrt(cfg.D)
    (q_idx, _, key, _, _), (qi_r, _, key_r, _, _) = _varlen_lists(ca, case)
    dev = [case[n].to(DEV) for n in ("q", "k", "v", "do")]
    plan = ca.bwd_plan_varlen(q_idx, key, case["lengths"])
    o, lse = ca.fwd_varlen(dev[0], dev[1], dev[2], q_idx, key, scale)
    g = ca.bwd_varlen(dev[0], dev[1], dev[2], o, dev[3], lse, q_idx, key, scale, plan=plan)
    torch.cuda.synchronize()
    one = lambda n: case[n][None]
    o_r, lse_r = O.attn_fwd_gathered(one("q"), one("k"), one("v"), qi_r[None], key_r[None], scale)
    g_r = O.attn_bwd_gathered(one("q"), one("k"), one("v"), one("do"), qi_r[None], key_r[None], scale)
    _check_all(o[None], lse[None], [t[None] for t in g], o_r, lse_r, g_r, TOL[cfg.dtype])


def test_varlen_backward_is_deterministic(ca):
    case = make_varlen_case("varlen_mixed")
    cfg = case["cfg"]
    (q_idx, _, key, _, _), _ = _varlen_lists(ca, case)
    dev = [case[n].to(DEV) for n in ("q", "k", "v", "do")]
    o, lse = ca.fwd_varlen(dev[0], dev[1], dev[2], q_idx, key)
    r1 = ca.bwd_varlen(dev[0], dev[1], dev[2], o, dev[3], lse, q_idx, key)
    r2 = ca.bwd_varlen(dev[0], dev[1], dev[2], o, dev[3], lse, q_idx, key)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
