"""Pins of the oracle's ragged geometry (a partial last cluster when 8 does
not divide N; packed batches of images of different sizes) against a
hand-worked example, an independent exact-rational brute force and the
definitions the packed form must reduce to (no GPU)."""

import functools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from gen import make_case, make_varlen_case


def _zorder_cmp(a, b):
    """Independent Z-order comparison of two fixed-point points (x in the
    even bits): the axis whose XOR has the highest set bit decides, y at
    equal bit level."""
    xx, yy = a[0] ^ b[0], a[1] ^ b[1]
    if xx == 0 and yy == 0:
        return 0
    if yy.bit_length() >= xx.bit_length():
        return -1 if a[1] < b[1] else 1
    return -1 if a[0] < b[0] else 1


def _brute_force(coords, G, k, cs=8):
    """Clusters and lists written from the definition with Python integers
    and Fractions: Morton order by comparator, runs of cs, mean of the
    members' fixed-point coordinates as an exact rational, neighbours by
    (exact squared mean distance, index)."""
    qx, qy = O.quantize(coords, G)
    pts = [(int(x), int(y)) for x, y in zip(qx, qy)]
    n = len(pts)
    order = sorted(range(n), key=functools.cmp_to_key(
        lambda i, j: _zorder_cmp(pts[i], pts[j]) or (i > j) - (i < j)))
    runs = [order[i:i + cs] for i in range(0, n, cs)]
    means = [(Fraction(sum(pts[t][0] for t in r), len(r)), Fraction(sum(pts[t][1] for t in r), len(r)))
             for r in runs]
    C = len(runs)
    nbr = []
    for c in range(C):
        d = sorted(((means[o][0] - means[c][0]) ** 2 + (means[o][1] - means[c][1]) ** 2, o)
                   for o in range(C) if o != c)
        row = [c] + [o for _, o in d[:k - 1]]
        nbr.append(row + [-1] * (k - len(row)))
    q_idx = [r + [-1] * (cs - len(r)) for r in runs]
    key_idx = [sum((q_idx[j] if j >= 0 else [-1] * cs for j in row), []) for row in nbr]
    return np.array(q_idx).reshape(-1, cs), np.array(nbr).reshape(-1, k), \
        np.array(key_idx).reshape(-1, k * cs)


def test_partial_cluster_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ragged_partial_cluster.json")))
    coords = np.array(g["coords"], dtype=np.float32)
    for k, key in ((g["k"], "nbr"), (3, "nbr_k3")):
        q_idx, nbr, key_idx = O.build_image(coords, g["grid_side"], k=k)
        assert nbr.tolist() == g[key]
        for c, cells in enumerate(g["clusters_xy"]):
            members = q_idx[c][q_idx[c] >= 0]
            assert sorted(coords[members].astype(int).tolist()) == cells
        assert q_idx[2].tolist()[4:] == [-1] * 4
        # the partial cluster's own slots: its 4 tokens, then 4 empty slots
        assert key_idx[2, :8].tolist() == q_idx[2].tolist()


@pytest.mark.parametrize("seed", range(6))
def test_ragged_build_matches_exact_rational_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    G = 16
    for _ in range(8):
        n = int(rng.integers(1, 70))
        pts = rng.uniform(-0.5, G - 0.5, size=(n, 2)).astype(np.float32)
        if seed % 2:                                  # repeated points: exact ties
            pts[n // 2:] = pts[: n - n // 2]
        k = int(rng.integers(1, 9))
        q_idx, nbr, key_idx = O.build_image(pts, G, k=k)
        bq, bn, bk = _brute_force(pts, G, k)
        assert np.array_equal(q_idx, bq)
        assert np.array_equal(nbr, bn), (n, k)
        assert np.array_equal(key_idx, bk)


def test_full_images_keep_the_plain_centroid_order():
    """When 8 divides N the scaled centroids are 105 times the plain sums:
    the same lists as the full-cluster rule."""
    for name in ("tiny", "stage3"):
        case = make_case(name, B=2, tensors=False)
        cfg = case["cfg"]
        for b in range(cfg.B):
            qx, qy = O.quantize(case["coords"][b], cfg.G)
            perm = O.balanced_clusters(O.morton_code(qx, qy))
            plain = O.nearest_clusters(O.centroid_sums(perm, qx, qy, 8), 6)
            q_idx, nbr, _ = O.build_image(case["coords"][b], cfg.G)
            assert np.array_equal(nbr, plain)
            assert np.array_equal(q_idx.reshape(-1), perm)


@pytest.mark.parametrize("name", ["stage2", "stage4"])
def test_partial_cluster_structure(name):
    case = make_case(name, B=2, tensors=False)
    cfg = case["cfg"]
    perm, nbr, key_idx = O.build_neighbors(case["coords"], cfg.G)
    assert perm.shape == (2, cfg.C * 8) and cfg.N % 8 != 0
    for b in range(2):
        q = perm[b]
        assert np.array_equal(np.sort(q[q >= 0]), np.arange(cfg.N))       # every token once
        assert (q[cfg.N:] == -1).all() and (q[:cfg.N] >= 0).all()          # padding only at the end
        assert (nbr[b, :, 0] == np.arange(cfg.C)).all()
        holes = (key_idx[b] == -1).sum(axis=1)
        # a list holds the partial cluster's 8 - N % 8 empty slots exactly when it lists it
        lists_p = (nbr[b] == cfg.C - 1).any(axis=1)
        assert np.array_equal(holes, np.where(lists_p, 8 - cfg.N % 8, 0))


def test_varlen_build_is_per_image_build_with_offsets():
    case = make_varlen_case("varlen_tiny", tensors=False)
    cfg = case["cfg"]
    q_idx, nbr, key_idx, tok_off, clu_off = O.build_neighbors_varlen(case["coords"], case["lengths"], cfg.G)
    assert q_idx.shape[0] == clu_off[-1] == sum(-(-n // 8) for n in case["lengths"])
    for b, n in enumerate(case["lengths"]):
        t0, c0, c1 = tok_off[b], clu_off[b], clu_off[b + 1]
        qi, nb, kl = O.build_image(case["coords"][t0:t0 + n], cfg.G)
        assert np.array_equal(q_idx[c0:c1], np.where(qi >= 0, qi + t0, -1))
        assert np.array_equal(nbr[c0:c1], np.where(nb >= 0, nb + c0, -1))
        assert np.array_equal(key_idx[c0:c1], np.where(kl >= 0, kl + t0, -1))
        # lists never leave their image
        live = key_idx[c0:c1][key_idx[c0:c1] >= 0]
        assert ((live >= t0) & (live < t0 + n)).all()


def _ragged_tensors(N, H, rng):
    pts = rng.uniform(0, 15, size=(1, N, 2)).astype(np.float32)
    perm, nbr, key_idx = O.build_neighbors(pts, 16, k=3)
    q_idx = perm.reshape(1, -1, 8)
    q, k, v, do = (rng.standard_normal((1, N, H, 32)) for _ in range(4))
    return q, k, v, do, q_idx, key_idx


def test_partial_cluster_dense_equals_gathered():
    rng = np.random.default_rng(7)
    q, k, v, do, q_idx, key_idx = _ragged_tensors(29, 2, rng)    # 3 full clusters + 5 members
    s = 0.3
    Od, Ld = O.attn_fwd_dense(q, k, v, q_idx, key_idx, s)
    Og, Lg = O.attn_fwd_gathered(q, k, v, q_idx, key_idx, s)
    assert np.isfinite(Ld).all() and np.allclose(Od, Og, atol=1e-12) and np.allclose(Ld, Lg, atol=1e-12)
    gd = O.attn_bwd_dense(q, k, v, do, q_idx, key_idx, s)
    gg = O.attn_bwd_gathered(q, k, v, do, q_idx, key_idx, s)
    for a, b in zip(gd, gg):
        assert np.allclose(a, b, atol=1e-12)


def test_partial_cluster_finite_differences():
    rng = np.random.default_rng(8)
    q, k, v, do, q_idx, key_idx = _ragged_tensors(13, 1, rng)    # one full cluster + 5 members
    s = 0.25
    dq, dk, dv = O.attn_bwd_gathered(q, k, v, do, q_idx, key_idx, s)

    def loss(q_, k_, v_):
        return float((O.attn_fwd_gathered(q_, k_, v_, q_idx, key_idx, s)[0] * do).sum())

    eps = 1e-6
    for name, X, G in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for t in (0, 6, 12):
            for d in (0, 17):
                Xp, Xm = X.copy(), X.copy()
                Xp[0, t, 0, d] += eps
                Xm[0, t, 0, d] -= eps
                args_p = {"q": (Xp, k, v), "k": (q, Xp, v), "v": (q, k, Xp)}[name]
                args_m = {"q": (Xm, k, v), "k": (q, Xm, v), "v": (q, k, Xm)}[name]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                assert abs(fd - G[0, t, 0, d]) < 1e-6 * max(1.0, abs(fd)), (name, t, d)


def test_varlen_attention_equals_separate_images():
    """The packed form (one index space with global ids) must give each
    image exactly what the image gives on its own."""
    case = make_varlen_case("varlen_tiny")
    cfg = case["cfg"]
    q_idx, nbr, key_idx, tok_off, _ = O.build_neighbors_varlen(case["coords"], case["lengths"], cfg.G)
    q, k, v, do = (case[n].double().numpy() for n in ("q", "k", "v", "do"))
    s = 1 / np.sqrt(32)
    Op, Lp = O.attn_fwd_gathered(q[None], k[None], v[None], q_idx[None], key_idx[None], s)
    gp = O.attn_bwd_gathered(q[None], k[None], v[None], do[None], q_idx[None], key_idx[None], s)
    for b, n in enumerate(case["lengths"]):
        if n == 0:
            continue
        t0 = tok_off[b]
        sl = slice(t0, t0 + n)
        qi, _, kl = O.build_image(case["coords"][sl], cfg.G)
        Oi, Li = O.attn_fwd_gathered(q[None, sl], k[None, sl], v[None, sl], qi[None], kl[None], s)
        assert np.array_equal(Op[0, sl], Oi[0]) and np.array_equal(Lp[0, sl], Li[0])
        gi = O.attn_bwd_gathered(q[None, sl], k[None, sl], v[None, sl], do[None, sl], qi[None], kl[None], s)
        for a, c in zip(gp, gi):
            assert np.allclose(a[0, sl], c[0], atol=1e-13)
