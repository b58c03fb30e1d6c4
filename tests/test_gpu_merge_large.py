"""GPU parity of adaptive token merging on whole fine-tune images (every
cell of a 128 x 128 or 256 x 256 token grid; images above 4096 tokens take
the global-memory plan), through the C ABI, against the fp64 oracle (its
k-d tree form of the nearest-anchor rule, pinned against the per-token
scan).  The plan must match exactly; merged features and gradients within
the bars of the small-image tests plus a term for fp32 sums over large
groups (up to thousands of members here)."""

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


_CASES = {}


def _case(name, B=None):
    key = (name, B)
    if key not in _CASES:
        _CASES[key] = make_merge_case(name, B=B)
    return _CASES[key]


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
    assign = O.merge_assign_tree(coords, anchors, G)
    N = assign.size
    members = np.lexsort((np.arange(N), assign))
    offsets = np.concatenate([[0], np.cumsum(np.bincount(assign, minlength=k))])
    return anchors, assign, members, offsets


def _plan_equal(ca_plan, b, ref):
    for name, g, r in zip(("anchors", "assign", "members", "offsets"), ca_plan, ref):
        gg = g[b].cpu().numpy()
        bad = np.argwhere(gg != r)
        assert bad.size == 0, f"image {b} {name}: {len(bad)} differ, first {bad[:3].ravel().tolist()}"


def _run(ca, coords, scores, feats, dfeat, dcoord, k, G, images=None):
    B, N, C = feats.shape
    dc = torch.from_numpy(coords).to(DEV)
    ds = torch.from_numpy(scores).to(DEV)
    plan = ca.merge_plan(dc, ds, k, G)
    _, _, members, offsets = plan
    f = feats.to(DEV)
    of, ox = ca.merge_fwd(f, dc, ds, members, offsets)
    dF, dX, dS = ca.merge_bwd(f, dc, ds, members, offsets, dfeat.to(DEV),
                              torch.from_numpy(dcoord).to(DEV))
    torch.cuda.synchronize()
    F64, dF64 = feats.double().numpy(), dfeat.double().numpy()
    for b in (range(B) if images is None else images):
        ref = _ref_plan(coords[b], scores[b], k, G)
        _plan_equal(plan, b, ref)
        rs = ref[1]
        # fp32 sums over a group of n members: the weights' normaliser and
        # the weighted sums each carry up to about n u of relative error
        # (u = 2^-24), bounded by (2 n + 8) u times the sum of the terms'
        # magnitudes; n is in the thousands in the one- and two-anchor cases
        gam = (2 * np.bincount(rs, minlength=k) + 8) * 2.0 ** -24
        w = O.merge_weights(scores[b], rs, k)
        X64 = coords[b].astype(np.float64)
        magF = np.zeros((k, C))
        np.add.at(magF, rs, w[:, None] * np.abs(F64[b]))
        magX = np.zeros((k, 2))
        np.add.at(magX, rs, w[:, None] * np.abs(X64))
        Fm, Xm = O.merge_fwd(F64[b], coords[b], scores[b], rs, k)
        _check(f"b{b} feats", of[b].double().cpu().numpy(), Fm,
               _bar(feats.dtype, Fm) + gam[:, None] * magF)
        _check(f"b{b} coords", ox[b].double().cpu().numpy(), Xm,
               2e-6 * np.abs(Xm) + 1e-5 + gam[:, None] * magX)
        rdF, rdX, rdS = O.merge_bwd(F64[b], coords[b], scores[b], rs, k, dF64[b], dcoord[b])
        gi = gam[rs][:, None]
        _check(f"b{b} dfeats", dF[b].double().cpu().numpy(), rdF,
               _bar(feats.dtype, rdF) + gi * np.abs(rdF))
        _check(f"b{b} dcoords", dX[b].double().cpu().numpy(), rdX,
               2e-6 * np.abs(rdX) + 1e-6 + gi * np.abs(rdX))
        sc = max(1.0, float(np.abs(rdS).max()))
        _check(f"b{b} dscores", dS[b].double().cpu().numpy(), rdS,
               1e-4 * sc + 1e-4 * np.abs(rdS) + gi[:, 0] * np.abs(rdS))
    return plan


@pytest.mark.parametrize("name,li", [("merge_finetune", 0), ("merge_finetune", 1),
                                     ("merge_finetune", 2), ("merge_highres", 0),
                                     ("merge_highres", 1), ("merge_highres", 2)])
def test_whole_grid_levels(ca, name, li):
    """The full four-image launches, every image compared in full."""
    case = _case(name)
    cfg = case["cfg"]
    N, k, C = cfg.levels[li]
    print(f"case {name} B={cfg.B} level {li} (N={N}, k={k}, C={C})", flush=True)
    _run(ca, case["coords"][li], case["scores"][li], case["feats"][li], case["dfeat"][li],
         case["dcoord"][li], k, cfg.G)


@pytest.mark.parametrize("N,k,G,scores", [(20000, 7777, 64, "ties"), (4097, 1, 64, "normal"),
                                         (5000, 5000, 64, "normal"), (9000, 2, 300, "ties"),
                                         (12000, 4000, 1, "normal"), (70000, 3, 256, "ties")])
def test_large_plan_edge_cases(ca, N, k, G, scores):
    """Scores with many ties across the select kernel's chunks (part of the
    tied value taken), one anchor (a single group of every token), every
    token an anchor, a grid side that is not a power of two, a one-cell
    grid (all coordinates quantised onto few points: distance ties), and
    three groups of ~23,000 members (their lists sorted by three radix
    passes)."""
    rng = np.random.default_rng(N + k + G)
    B, C = 2, 16
    X = rng.uniform(-1.0, G, size=(B, N, 2)).astype(np.float32)
    X[:, N // 2:N // 2 + N // 4] = X[:, :N // 4]
    if scores == "ties":
        S = rng.integers(-3, 3, size=(B, N)).astype(np.float32)
    else:
        S = rng.standard_normal((B, N)).astype(np.float32)
    F = torch.from_numpy(rng.standard_normal((B, N, C)).astype(np.float32))
    dF = torch.from_numpy(rng.standard_normal((B, k, C)).astype(np.float32))
    dX = rng.standard_normal((B, k, 2)).astype(np.float32)
    print(f"case merge large edge N={N} k={k} G={G} scores={scores}", flush=True)
    _run(ca, X, S, F, dF, dX, k, G)


def test_large_plan_repeats_bitwise(ca):
    """The plan's placement runs on integer atomics; its outputs must not
    depend on their order."""
    case = _case("merge_highres")
    cfg = case["cfg"]
    N, k, _ = cfg.levels[0]
    dc = torch.from_numpy(case["coords"][0]).to(DEV)
    ds = torch.from_numpy(case["scores"][0]).to(DEV)
    p1 = ca.merge_plan(dc, ds, k, cfg.G)
    p2 = ca.merge_plan(dc, ds, k, cfg.G)
    for a, b in zip(p1, p2):
        assert torch.equal(a, b)
