"""GPU parity of adaptive token merging against the fp64 oracle, through the
C ABI.  The plan (anchors, assignment, member lists) must match exactly;
merged features and gradients within bars derived from the arithmetic (fp32
accumulation, one RNE rounding of bf16 outputs: relative 2^-9)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gen import make_merge_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ca():
    import gathered_local_attention_amd as ca

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ca._lib.load()
    return ca


def _bar(dtype, ref):
    rel = {torch.float32: 2e-6, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[dtype]
    return rel * np.abs(ref) + 2e-5 * max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)


def _check(name, got, ref, bar):
    err = np.abs(got - ref)
    worst = float((err - bar).max()) if err.size else -1.0
    print(f"  {name}: max abs err {float(err.max()) if err.size else 0:.3e}", flush=True)
    assert worst <= 0, f"{name}: error above bar by {worst:.3e}"


def _ref_plan(coords, scores, k, G):
    anchors = O.merge_anchors(scores, k)
    assign = O.merge_assign(coords, anchors, G)
    N = assign.size
    members = np.lexsort((np.arange(N), assign))
    offsets = np.concatenate([[0], np.cumsum(np.bincount(assign, minlength=k))])
    return anchors, assign, members, offsets


def _run(ca, coords, scores, feats, dfeat, dcoord, k, G, images=None):
    B, N, C = feats.shape
    dc = torch.from_numpy(coords).to(DEV)
    ds = torch.from_numpy(scores).to(DEV)
    anchors, assign, members, offsets = ca.merge_plan(dc, ds, k, G)
    f = feats.to(DEV)
    of, ox = ca.merge_fwd(f, dc, ds, members, offsets)
    dF, dX, dS = ca.merge_bwd(f, dc, ds, members, offsets, dfeat.to(DEV), torch.from_numpy(dcoord).to(DEV))
    torch.cuda.synchronize()
    F64 = feats.double().numpy()
    dF64 = dfeat.double().numpy()
    for b in (range(B) if images is None else images):
        ra, rs, rm, ro = _ref_plan(coords[b], scores[b], k, G)
        for name, g, r in (("anchors", anchors, ra), ("assign", assign, rs), ("members", members, rm),
                           ("offsets", offsets, ro)):
            gg = g[b].cpu().numpy()
            assert np.array_equal(gg, r), f"image {b} {name}: {np.argwhere(gg != r)[:3].tolist()}"
        Fm, Xm = O.merge_fwd(F64[b], coords[b], scores[b], rs, k)
        _check(f"b{b} feats", of[b].double().cpu().numpy(), Fm, _bar(feats.dtype, Fm))
        _check(f"b{b} coords", ox[b].double().cpu().numpy(), Xm, 2e-6 * np.abs(Xm) + 1e-5)
        rdF, rdX, rdS = O.merge_bwd(F64[b], coords[b], scores[b], rs, k, dF64[b], dcoord[b])
        _check(f"b{b} dfeats", dF[b].double().cpu().numpy(), rdF, _bar(feats.dtype, rdF))
        _check(f"b{b} dcoords", dX[b].double().cpu().numpy(), rdX, 2e-6 * np.abs(rdX) + 1e-6)
        sc = max(1.0, float(np.abs(rdS).max()))
        _check(f"b{b} dscores", dS[b].double().cpu().numpy(), rdS, 1e-4 * sc + 1e-4 * np.abs(rdS))
    return dF, dX, dS


@pytest.mark.parametrize("li", [0, 1])
def test_tiny_fp32(ca, li):
    case = make_merge_case("merge_tiny")
    cfg = case["cfg"]
    N, k, C = cfg.levels[li]
    print(f"case merge_tiny level {li}", flush=True)
    _run(ca, case["coords"][li], case["scores"][li], case["feats"][li], case["dfeat"][li],
         case["dcoord"][li], k, cfg.G)


@pytest.mark.parametrize("li", [0, 1, 2])
def test_stage_levels_bf16(ca, li):
    case = make_merge_case("merge_stages", B=2)
    cfg = case["cfg"]
    N, k, C = cfg.levels[li]
    print(f"case merge_stages B=2 level {li}", flush=True)
    _run(ca, case["coords"][li], case["scores"][li], case["feats"][li], case["dfeat"][li],
         case["dcoord"][li], k, cfg.G)


def test_full_batch_sampled_images(ca):
    case = make_merge_case("merge_stages")
    cfg = case["cfg"]
    for li, (N, k, C) in enumerate(cfg.levels):
        print(f"case merge_stages B=32 level {li} images 0, 31", flush=True)
        _run(ca, case["coords"][li], case["scores"][li], case["feats"][li], case["dfeat"][li],
             case["dcoord"][li], k, cfg.G, images=[0, 31])


@pytest.mark.parametrize("N,k", [(300, 300), (300, 1), (4096, 1638), (1, 1)])
def test_edge_sizes_and_ties(ca, N, k):
    """Every token an anchor, one anchor for all, the largest image, one
    token; integer scores (ties) and repeated coordinates."""
    rng = np.random.default_rng(N + k)
    G = 64
    coords = rng.uniform(-2, G + 1, size=(2, N, 2)).astype(np.float32)
    coords[:, N // 2:] = coords[:, : N - N // 2]
    scores = rng.integers(-3, 3, size=(2, N)).astype(np.float32)
    C = 16
    feats = torch.from_numpy(rng.standard_normal((2, N, C)).astype(np.float32))
    dfeat = torch.from_numpy(rng.standard_normal((2, k, C)).astype(np.float32))
    dcoord = rng.standard_normal((2, k, 2)).astype(np.float32)
    print(f"case merge edge N={N} k={k}", flush=True)
    _run(ca, coords, scores, feats, dfeat, dcoord, k, G)


@pytest.mark.parametrize("dtype,N,k,C", [(torch.float16, 400, 100, 192),
                                         (torch.bfloat16, 300, 60, 768),
                                         (torch.float32, 200, 50, 1024),
                                         (torch.bfloat16, 150, 7, 1024),
                                         (torch.float32, 100, 100, 8)])
def test_row_widths_all_dtypes(ca, dtype, N, k, C):
    """Every element type and row width: one to four 16-byte chunks per lane,
    groups where some lanes hold one chunk fewer (768 bf16 channels), idle
    lanes (192 f16 channels over 32 lanes), groups of one member and groups
    of tens of members (several batches of four)."""
    rng = np.random.default_rng(N * 31 + C)
    G = 32
    coords = rng.uniform(-0.5, G - 0.5, size=(2, N, 2)).astype(np.float32)
    scores = rng.standard_normal((2, N)).astype(np.float32)
    feats = torch.from_numpy(rng.standard_normal((2, N, C)).astype(np.float32)).to(dtype)
    dfeat = torch.from_numpy(rng.standard_normal((2, k, C)).astype(np.float32)).to(dtype)
    dcoord = rng.standard_normal((2, k, 2)).astype(np.float32)
    print(f"case merge widths dtype={dtype} N={N} k={k} C={C}", flush=True)
    _run(ca, coords, scores, feats, dfeat, dcoord, k, G)


def test_backward_is_deterministic(ca):
    case = make_merge_case("merge_stages", B=4)
    cfg = case["cfg"]
    N, k, C = cfg.levels[0]
    dc = torch.from_numpy(case["coords"][0]).to(DEV)
    ds = torch.from_numpy(case["scores"][0]).to(DEV)
    _, _, members, offsets = ca.merge_plan(dc, ds, k, cfg.G)
    f = case["feats"][0].to(DEV)
    args = (f, dc, ds, members, offsets, case["dfeat"][0].to(DEV), torch.from_numpy(case["dcoord"][0]).to(DEV))
    r1, r2 = ca.merge_bwd(*args), ca.merge_bwd(*args)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
