"""Pins of the oracle's 3D neighbour build against closed forms, an
independent exact-rational brute force and the 2D build it reduces to
(no GPU)."""

import functools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from gen import make_volume_case


def test_morton3_and_quantize_closed_forms(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "morton3_codes.json")))
    for c in g["morton"]:
        assert int(O.morton_code3(*(np.int64(v) for v in c["q"]))) == c["code"], c
    for c in g["quantize"]:
        qx, _, _ = O.quantize3(np.array([[c["c"], 0.0, 0.0]], dtype=np.float32), c["G"])
        assert int(qx[0]) == c["q"], c


def _z3_cmp(a, b):
    """Independent 3D Z-order comparison: the axis whose XOR has the highest
    set bit decides; at equal bit level z beats y beats x."""
    xs = [a[i] ^ b[i] for i in range(3)]
    lv = [v.bit_length() for v in xs]
    if max(lv) == 0:
        return 0
    top = max(i for i in range(3) if lv[i] == max(lv))
    return -1 if a[top] < b[top] else 1


def _brute3(coords, G, k, cs=8):
    qx, qy, qz = O.quantize3(coords, G)
    pts = [(int(x), int(y), int(z)) for x, y, z in zip(qx, qy, qz)]
    n = len(pts)
    order = sorted(range(n), key=functools.cmp_to_key(
        lambda i, j: _z3_cmp(pts[i], pts[j]) or (i > j) - (i < j)))
    runs = [order[i:i + cs] for i in range(0, n, cs)]
    means = [tuple(Fraction(sum(pts[t][a] for t in r), len(r)) for a in range(3)) for r in runs]
    nbr = []
    for c in range(len(runs)):
        d = sorted((sum((means[o][a] - means[c][a]) ** 2 for a in range(3)), o)
                   for o in range(len(runs)) if o != c)
        row = [c] + [o for _, o in d[:k - 1]]
        nbr.append(row + [-1] * (k - len(row)))
    return [r + [-1] * (cs - len(r)) for r in runs], nbr


@pytest.mark.parametrize("seed", range(5))
def test_build3_matches_exact_rational_brute_force(seed):
    rng = np.random.default_rng(300 + seed)
    G = 16
    for _ in range(6):
        n = int(rng.integers(1, 90))
        pts = rng.uniform(-0.5, G - 0.5, size=(n, 3)).astype(np.float32)
        if seed % 2:
            pts[n // 2:] = pts[: n - n // 2]          # repeated points: exact ties
        k = int(rng.integers(1, 9))
        q_idx, nbr, key_idx = O.build_image3(pts, G, k=k)
        bq, bn = _brute3(pts, G, k)
        assert q_idx.tolist() == bq and nbr.tolist() == bn, (n, k)
        for c in range(nbr.shape[0]):
            expect = sum((bq[j] if j >= 0 else [-1] * 8 for j in bn[c]), [])
            assert key_idx[c].tolist() == expect


def test_full_grid_clusters_are_cubes_and_face_neighbours():
    """On the full 4x4x4 integer grid every cluster is a 2x2x2 block (block
    (X, Y, Z) is cluster X + 2Y + 4Z); its three face neighbours (one axis
    flipped: c^1, c^2, c^4) are at distance 2, the three edge neighbours
    (c^3, c^5, c^6) at 2*sqrt(2), ties by index."""
    G = 4
    cells = np.random.default_rng(1).permutation(G ** 3)
    xyz = np.stack([cells % G, (cells // G) % G, cells // (G * G)], 1).astype(np.float32)
    q_idx, nbr, _ = O.build_image3(xyz, G, k=6)
    for c in range(8):
        X, Y, Z = c & 1, (c >> 1) & 1, c >> 2
        members = xyz[q_idx[c]].astype(int)
        assert sorted(map(tuple, members)) == sorted(
            (2 * X + dx, 2 * Y + dy, 2 * Z + dz) for dx in (0, 1) for dy in (0, 1) for dz in (0, 1))
        assert tuple(members[0]) == (2 * X, 2 * Y, 2 * Z) and tuple(members[7]) == (2 * X + 1, 2 * Y + 1, 2 * Z + 1)
        assert nbr[c].tolist() == [c] + sorted([c ^ 1, c ^ 2, c ^ 4]) + sorted([c ^ 3, c ^ 5, c ^ 6])[:2]


def test_flat_volume_reduces_to_the_2d_build():
    """Integer points with z = 0: both quantisations are exact affine maps and
    the 3D interleave keeps the relative order of the x and y bits, so the
    clusters and lists equal the 2D build's."""
    rng = np.random.default_rng(4)
    for n in (256, 203):
        cells = rng.choice(32 * 32, size=n, replace=False)
        xy = np.stack([cells % 32, cells // 32], 1).astype(np.float32)
        xyz = np.concatenate([xy, np.zeros((n, 1), np.float32)], 1)
        q3, n3, k3 = O.build_image3(xyz, 32)
        q2, n2, k2 = O.build_image(xy, 32)
        assert np.array_equal(q3, q2) and np.array_equal(n3, n2) and np.array_equal(k3, k2)


def test_volume_workload_lists_are_valid():
    case = make_volume_case("volume", B=2, tensors=False)
    cfg = case["cfg"]
    perm, nbr, key_idx = O.build_neighbors_3d(case["coords"], cfg.G)
    for b in range(2):
        assert np.array_equal(np.sort(perm[b]), np.arange(cfg.N))
        assert (nbr[b, :, 0] == np.arange(cfg.N // 8)).all()
        assert all(len(set(r)) == 48 for r in key_idx[b])


def test_packed_volumes_are_per_volume_builds():
    case = make_volume_case("volume_varlen", B=3, tensors=False)
    cfg = case["cfg"]
    q_idx, nbr, key_idx, tok_off, clu_off = O.build_neighbors_varlen_3d(case["coords"], case["lengths"], cfg.G)
    for b, n in enumerate(case["lengths"]):
        qi, nb, kl = O.build_image3(case["coords"][tok_off[b]:tok_off[b + 1]], cfg.G)
        c0, c1 = clu_off[b], clu_off[b + 1]
        assert np.array_equal(q_idx[c0:c1], np.where(qi >= 0, qi + tok_off[b], -1))
        assert np.array_equal(nbr[c0:c1], np.where(nb >= 0, nb + c0, -1))
        assert np.array_equal(key_idx[c0:c1], np.where(kl >= 0, kl + tok_off[b], -1))
