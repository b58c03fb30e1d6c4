"""GPU parity of the 3D (volumetric) neighbour build against the fp64/integer
oracle, through the C ABI (lists bit-exact), and of the attention over 3D
lists (tolerances of ``parity_util``)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from gen import make_volume_case
from parity_util import TOL, assert_finite, check_close, sampled_oracle, to_np

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


def _lists(ca, coords, G, k=6):
    got = ca.build_neighbors(torch.from_numpy(coords).to(DEV), G, k=k)
    ref = O.build_neighbors_3d(coords, G, k=k)
    for nm, g, r in zip(("perm", "nbr", "key_idx"), got, ref):
        _equal(nm, g, r)
    return got, ref


@pytest.mark.parametrize("name", ["vol_tiny", "volume", "volume_hr"])
def test_volume_lists_bit_exact(ca, name):
    case = make_volume_case(name, tensors=False)
    cfg = case["cfg"]
    print(f"case {name} B={cfg.B} N={cfg.N} G={cfg.G}", flush=True)
    _lists(ca, case["coords"], cfg.G)


@pytest.mark.parametrize("N,k", [(1, 6), (13, 2), (2049, 6), (4100, 4), (6001, 8)])
def test_volume_lists_ragged_and_ties(ca, N, k):
    """Every path (in-LDS 2048 / 4096, segments) with a partial last
    cluster; repeated points give exact code and distance ties."""
    rng = np.random.default_rng(N * 7 + k)
    G = 24
    coords = rng.uniform(-0.5, G - 0.5, size=(2, N, 3)).astype(np.float32)
    coords[1, N // 2:] = coords[1, : N - N // 2]
    print(f"case volume ragged N={N} k={k}", flush=True)
    _lists(ca, coords, G, k=k)


def test_packed_volumes_bit_exact(ca):
    case = make_volume_case("volume_varlen", tensors=False)
    cfg = case["cfg"]
    print(f"case volume_varlen lengths {case['lengths']}", flush=True)
    got = ca.build_neighbors_varlen(torch.from_numpy(case["coords"]).to(DEV), case["lengths"], cfg.G)
    ref = O.build_neighbors_varlen_3d(case["coords"], case["lengths"], cfg.G)
    for nm, g, r in zip(("q_idx", "nbr", "key_idx", "tok_off", "clu_off"), got, ref):
        _equal(nm, g, r.astype(np.int32))


@pytest.mark.parametrize("name,B", [("vol_tiny", None), ("volume", 2)])
def test_attention_on_volume_lists(ca, name, B):
    case = make_volume_case(name, B=B)
    cfg = case["cfg"]
    print(f"case {name} attention B={cfg.B} {cfg.dtype}", flush=True)
    scale = 1.0 / math.sqrt(cfg.D)
    (perm, _, key), (perm_r, _, key_r) = _lists(ca, case["coords"], cfg.G)
    qi_r = perm_r.reshape(cfg.B, -1, 8)
    dev = [case[n].to(DEV) for n in ("q", "k", "v", "do")]
    o, lse = ca.fwd(dev[0], dev[1], dev[2], perm, key, scale)
    g = ca.bwd(dev[0], dev[1], dev[2], o, dev[3], lse, perm, key, scale)
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    o_r, lse_r = O.attn_fwd_gathered(case["q"], case["k"], case["v"], qi_r, key_r, scale)
    g_r = O.attn_bwd_gathered(case["q"], case["k"], case["v"], case["do"], qi_r, key_r, scale)
    for nm, t in (("O", o), ("LSE", lse)) + tuple(zip(("dQ", "dK", "dV"), g)):
        assert_finite(nm, t)
    check_close("O", o, o_r, tol["o"], False)
    check_close("LSE", lse, lse_r, tol["lse"], False)
    for nm, a, r in zip(("dQ", "dK", "dV"), g, g_r):
        check_close(nm, a, r, tol["g"], False)


def test_volume_full_batch_sampled(ca):
    """The 32-volume batch as the benchmark runs it: sampled outputs."""
    case = make_volume_case("volume")
    cfg = case["cfg"]
    scale = 1.0 / math.sqrt(cfg.D)
    print("case volume full", flush=True)
    (perm, _, key), (perm_r, _, key_r) = _lists(ca, case["coords"], cfg.G)
    dev = [case[n].to(DEV) for n in ("q", "k", "v", "do")]
    o, lse = ca.fwd(dev[0], dev[1], dev[2], perm, key, scale)
    dq, dk, dv = ca.bwd(dev[0], dev[1], dev[2], o, dev[3], lse, perm, key, scale)
    torch.cuda.synchronize()
    tol = TOL[cfg.dtype]
    rng = np.random.default_rng(97)
    qi = perm_r.reshape(cfg.B, -1, 8)
    for b in (3, 30):
        clusters = np.sort(rng.choice(qi.shape[1], 24, replace=False))
        key_tokens = np.sort(rng.choice(cfg.N, 48, replace=False))
        one = lambda n: case[n][b:b + 1]
        ref = sampled_oracle(one("q"), one("k"), one("v"), one("do"), qi[b], key_r[b], scale,
                             clusters, key_tokens)
        tq, tk = ref["q_tokens"], ref["k_tokens"]
        check_close("O", to_np(o[b, tq]), ref["o"], tol["o"], False)
        check_close("LSE", to_np(lse[b, tq]), ref["lse"], tol["lse"], False)
        check_close("dQ", to_np(dq[b, tq]), ref["dq"], tol["g"], False)
        check_close("dK", to_np(dk[b, tk]), ref["dk"], tol["g"], False)
        check_close("dV", to_np(dv[b, tk]), ref["dv"], tol["g"], False)
