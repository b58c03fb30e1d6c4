"""Pins of the oracle's neighbour build against closed forms, hand-worked
examples and independent brute force (no GPU)."""

import functools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from gen import make_case


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_morton_closed_forms(golden_dir):
    g = _load(golden_dir, "morton_codes.json")
    for c in g["cases"]:
        assert int(O.morton_code(np.int64(c["qx"]), np.int64(c["qy"]))) == c["code"], c


def test_quantize_closed_forms(golden_dir):
    g = _load(golden_dir, "morton_codes.json")["quantize"]
    for c in g["cases"]:
        xy = np.array([[c["c"], 0.0]], dtype=np.float32)
        qx, _ = O.quantize(xy, c["G"])
        assert int(qx[0]) == c["q"], c


def _zorder_less(a, b):
    """Independent Z-order comparator: the axis whose XOR has the highest set
    bit decides; at equal bit level y is the more significant (odd bits)."""
    ax, ay = int(a[0]), int(a[1])
    bx, by = int(b[0]), int(b[1])
    xx, yy = ax ^ bx, ay ^ by
    if xx == 0 and yy == 0:
        return 0
    if yy.bit_length() >= xx.bit_length():
        return -1 if ay < by else 1
    return -1 if ax < bx else 1


def test_sort_matches_independent_zorder():
    rng = np.random.default_rng(5)
    for trial in range(20):
        n = 64
        q = rng.integers(0, 65536, size=(n, 2))
        if trial % 2:          # force ties and shared prefixes
            q = q // 4096 * 4096
        code = O.morton_code(q[:, 0], q[:, 1])
        perm = O.balanced_clusters(code)
        keyed = sorted(range(n), key=functools.cmp_to_key(
            lambda i, j: _zorder_less(tuple(q[i]), tuple(q[j])) or (i > j) - (i < j)))
        assert list(perm) == keyed


def _grid_coords(G, order=None):
    cells = np.arange(G * G) if order is None else order
    return np.stack([cells % G, cells // G], axis=1).astype(np.float32)[None]


@pytest.mark.parametrize("shuffle", [False, True])
def test_full_grid_clusters_are_4x2_blocks(shuffle):
    G = 32
    order = np.random.default_rng(3).permutation(G * G) if shuffle else None
    coords = _grid_coords(G, order)
    perm, nbr, key_idx = O.build_neighbors(coords, G)
    xy = coords[0][perm[0]].astype(int)
    for c in range(G * G // 8):
        bits = [(c >> i) & 1 for i in range(7)]
        Y = bits[0] + 2 * bits[2] + 4 * bits[4] + 8 * bits[6]
        X = bits[1] + 2 * bits[3] + 4 * bits[5]
        members = xy[8 * c: 8 * c + 8]
        expect = [(4 * X + dx, 2 * Y + dy) for dy in range(2) for dx in range(4)]
        assert sorted(map(tuple, members)) == sorted(expect)
        # inside a cluster the members stay in Morton order
        first = [(4 * X, 2 * Y), (4 * X + 1, 2 * Y), (4 * X, 2 * Y + 1), (4 * X + 1, 2 * Y + 1)]
        assert [tuple(m) for m in members[:4]] == first


def test_grid32_worked_neighbour_example(golden_dir):
    g = _load(golden_dir, "grid32_cluster24.json")
    coords = _grid_coords(g["grid_side"])
    perm, nbr, key_idx = O.build_neighbors(coords, g["grid_side"])
    assert list(nbr[0, g["cluster"]]) == g["nbr"]
    mem = coords[0][perm[0][8 * g["cluster"]: 8 * g["cluster"] + 8]]
    assert list(mem.mean(axis=0)) == g["centroid"]
    # key list = concatenated members of the listed clusters, in order
    for s, c in enumerate(g["nbr"]):
        assert list(key_idx[0, g["cluster"], 8 * s: 8 * s + 8]) == list(perm[0][8 * c: 8 * c + 8])


@pytest.mark.parametrize("name,B", [("tiny", None), ("stage1", 1), ("stage3", 2)])
def test_partial_selection_equals_full_sort(name, B):
    case = make_case(name, B=B, tensors=False)
    cfg = case["cfg"]
    for b in range(cfg.B):
        qx, qy = O.quantize(case["coords"][b], cfg.G)
        perm = O.balanced_clusters(O.morton_code(qx, qy))
        S = O.centroid_sums(perm, qx, qy, 8)
        assert np.array_equal(O.nearest_clusters(S, 6), O.nearest_clusters_fullsort(S, 6))


@pytest.mark.parametrize("name,B", [("tiny", None), ("stage1", 1)])
def test_neighbours_match_exact_rational_euclid(name, B):
    """On integer coordinates the fixed-point sums are an affine image of the
    true means with the same factor on both axes, so the order must equal the
    exact Euclidean order of the f32 coordinate means (computed with
    Fractions, no quantisation at all)."""
    case = make_case(name, B=B, tensors=False)
    cfg = case["cfg"]
    perm, nbr, _ = O.build_neighbors(case["coords"], cfg.G)
    for b in range(cfg.B):
        pts = case["coords"][b]
        C = cfg.C
        means = []
        for c in range(C):
            m = perm[b][8 * c: 8 * c + 8]
            means.append((sum(Fraction(float(x)) for x in pts[m, 0]) / 8,
                          sum(Fraction(float(y)) for y in pts[m, 1]) / 8))
        for c in range(0, C, max(1, C // 24)):
            d = sorted(((means[o][0] - means[c][0]) ** 2 + (means[o][1] - means[c][1]) ** 2, o)
                       for o in range(C) if o != c)
            assert list(nbr[b, c]) == [c] + [o for _, o in d[:5]]


def test_cluster_sets_follow_token_relabelling():
    """Relabelling tokens together with their coordinates gives the same
    clusters (as coordinate sets) when the Morton codes have no ties."""
    case = make_case("stage3", B=2, tensors=False)
    cfg = case["cfg"]
    rng = np.random.default_rng(11)
    for b in range(cfg.B):
        coords = case["coords"][b:b + 1]
        qx, qy = O.quantize(coords[0], cfg.G)
        assert np.unique(O.morton_code(qx, qy)).size == cfg.N
        pi = rng.permutation(cfg.N)
        p1, n1, k1 = O.build_neighbors(coords, cfg.G)
        p2, n2, k2 = O.build_neighbors(coords[:, pi], cfg.G)
        assert np.array_equal(pi[p2[0]], p1[0])
        assert np.array_equal(n1, n2)
        assert np.array_equal(pi[np.where(k2 >= 0, k2, 0)], np.where(k1 >= 0, k1, 0))


def test_few_clusters_pad_with_minus_one():
    coords = _grid_coords(4)[:, :16]          # 16 tokens -> 2 clusters
    perm, nbr, key_idx = O.build_neighbors(coords, 4)
    assert list(nbr[0, 0]) == [0, 1, -1, -1, -1, -1]
    assert list(nbr[0, 1]) == [1, 0, -1, -1, -1, -1]
    assert (key_idx[0, :, 16:] == -1).all()


def test_lists_are_valid_on_all_geometries():
    for name, B in (("tiny", None), ("stage1", 2), ("stage3", 2)):
        case = make_case(name, B=B, tensors=False)
        cfg = case["cfg"]
        perm, nbr, key_idx = O.build_neighbors(case["coords"], cfg.G)
        for b in range(cfg.B):
            assert np.array_equal(np.sort(perm[b]), np.arange(cfg.N))
            assert (nbr[b, :, 0] == np.arange(cfg.C)).all()
            for c in range(cfg.C):
                assert len(set(nbr[b, c])) == 6
                assert len(set(key_idx[b, c])) == 48
