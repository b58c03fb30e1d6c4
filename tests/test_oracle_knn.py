"""Pins of the KNN-cache point sampler oracle (no GPU): hand-worked tables,
closed forms of the weighting, an independent k-d tree search, and finite
differences of the forward for every gradient."""

import math

import numpy as np
import pytest

import oracle as O
from gen import make_sampler_case


def _table(points, G, K):
    return O.knn_table(np.asarray(points, dtype=np.float32), G, K)


def test_table_hand_worked_ties():
    """Reading K2 on three tokens of a 4x4 grid (worked by hand): tokens
    0 = (1, 0), 1 = (0, 1), 2 = (2, 2); equal distances go to the lower
    index.  Cells are (row, column) with centre (x = column, y = row)."""
    t = _table([[1, 0], [0, 1], [2, 2]], 4, 2)
    assert t[0, 0].tolist() == [0, 1]      # d2 1, 1 (tie), 8
    assert t[1, 1].tolist() == [0, 1]      # d2 1, 1 (tie), 2
    assert t[2, 2].tolist() == [2, 0]      # d2 5, 5 (tie), 0
    assert t[0, 2].tolist() == [0, 2]      # d2 1, 5, 4
    assert t[2, 0].tolist() == [1, 2]      # d2 5, 1, 4
    assert t[3, 3].tolist() == [2, 0]      # d2 13, 13 (tie), 2
    # fewer tokens than slots: -1 pads
    t3 = _table([[1, 0], [0, 1], [2, 2]], 4, 5)
    assert t3[0, 0].tolist() == [0, 1, 2, -1, -1]


def test_table_cells_hand_worked_and_padding():
    """The cell-restricted ranking on the hand-worked example above, in a
    shuffled cell order, and with more slots than tokens."""
    pts = np.asarray([[1, 0], [0, 1], [2, 2]], dtype=np.float32)
    rows = np.array([2, 0, 3, 1, 2, 0])
    cols = np.array([2, 0, 3, 1, 0, 2])
    got = O.knn_table_cells(pts, 4, 2, rows, cols)
    assert got.tolist() == [[2, 0], [0, 1], [2, 0], [0, 1], [1, 2], [0, 2]]
    assert O.knn_table_cells(pts, 4, 5, [0], [0]).tolist() == [[0, 1, 2, -1, -1]]
    assert O.knn_table_cells(np.zeros((0, 2), np.float32), 4, 3, [1], [2]).tolist() == [[-1] * 3]


@pytest.mark.parametrize("G,N,K,chunk", [(16, 150, 6, 7), (32, 600, 8, 256), (8, 5, 8, 3)])
def test_table_cells_match_full_table(G, N, K, chunk):
    """Every cell, in chunks that do not divide the cell count, against the
    per-cell lexicographic ranking (repeated coordinates give ties)."""
    rng = np.random.default_rng(G + N)
    pts = rng.uniform(-0.5, G - 0.5, size=(N, 2)).astype(np.float32)
    pts[N // 2:N // 2 + N // 5] = pts[:N // 5]
    full = O.knn_table(pts, G, K)
    ii, jj = np.meshgrid(np.arange(G), np.arange(G), indexing="ij")
    got = O.knn_table_cells(pts, G, K, ii.reshape(-1), jj.reshape(-1), chunk=chunk)
    np.testing.assert_array_equal(got, full.reshape(G * G, K))


def test_query_cells_closed_forms():
    q = np.array([[0.49, 0.5], [-3.0, 100.0], [2.5, 1.4999], [3.49, -0.5]], dtype=np.float32)
    i, j = O.query_cells(q, 4)
    assert j.tolist() == [0, 0, 3, 3]      # floor(x + 1/2), clamped to [0, 3]
    assert i.tolist() == [1, 3, 1, 0]


def test_table_matches_kdtree():
    """Independent search: scipy's k-d tree over the fixed-point coordinates
    (integers, exact in fp64), tie-aware comparison of each cell's list."""
    from scipy.spatial import cKDTree

    rng = np.random.default_rng(5)
    G, K = 16, 6
    pts = rng.uniform(-0.5, G - 0.5, size=(150, 2)).astype(np.float32)
    pts[100:110] = pts[:10]                # repeated coordinates: ties
    table = O.knn_table(pts, G, K)
    qx, qy = O.quantize(pts, G)
    P = np.stack([qx, qy], 1).astype(np.float64)
    tree = cKDTree(P)
    s = 2 ** (16 - 4)
    for i in range(G):
        for j in range(G):
            c = np.array([(j + 0.5) * s, (i + 0.5) * s])
            dk, _ = tree.query(c, k=K)
            rK = dk[-1]
            inside = np.array(sorted(tree.query_ball_point(c, rK * (1 + 1e-12) + 1e-9)))
            d2 = ((P[inside] - c) ** 2).sum(1)
            d2K = round(rK * rK)
            strict = inside[d2 < d2K - 0.5]
            ties = inside[np.abs(d2 - d2K) < 0.5]
            expect_set = set(strict.tolist()) | set(sorted(ties.tolist())[: K - strict.size])
            row = table[i, j].tolist()
            assert set(row) == expect_set, (i, j)
            rd2 = [((P[t] - c) ** 2).sum() for t in row]
            assert all((rd2[a], row[a]) < (rd2[a + 1], row[a + 1]) for a in range(K - 1)), (i, j)


def _small_case(seed=7, G=8, N=20, M=12, K=4, Cf=5, interior=True):
    rng = np.random.default_rng(seed)
    pts = rng.uniform(-0.5, G - 0.5, size=(N, 2)).astype(np.float32)
    cells = rng.integers(0, G, size=(M, 2))
    off = rng.uniform(-0.3, 0.3, size=(M, 2)) if interior else rng.uniform(-0.5, 0.5, size=(M, 2))
    q = (cells + off).astype(np.float32)
    F = rng.standard_normal((N, Cf))
    dO = rng.standard_normal((M, Cf))
    table = O.knn_table(pts, G, K)
    return pts, q, F, dO, table


def test_weights_closed_forms():
    pts, q, F, _, table = _small_case()
    slots, d, w = O.knn_weights(pts, q, table, 1.3)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    # ratios w_a / w_b = exp(-p (d_a - d_b)), distances from math.hypot
    for m in range(q.shape[0]):
        da = math.hypot(float(q[m, 0]) - float(pts[slots[m, 0], 0]), float(q[m, 1]) - float(pts[slots[m, 0], 1]))
        db = math.hypot(float(q[m, 0]) - float(pts[slots[m, 2], 0]), float(q[m, 1]) - float(pts[slots[m, 2], 1]))
        assert w[m, 0] / w[m, 2] == pytest.approx(math.exp(-1.3 * (da - db)), rel=1e-12)
    # p = 0: the plain mean of the slot rows
    out0 = O.knn_sample_fwd(pts, F, q, table, 0.0)
    assert np.allclose(out0, F[slots].mean(axis=1), rtol=0, atol=1e-14)
    # one slot: the row itself for any p
    t1 = O.knn_table(pts, 8, 1)
    out1 = O.knn_sample_fwd(pts, F, q, t1, 3.7)
    i, j = O.query_cells(q, 8)
    assert np.array_equal(out1, F[t1[i, j, 0]])
    # large p: the nearest slot dominates
    outL = O.knn_sample_fwd(pts, F, q, table, 400.0)
    near = slots[np.arange(len(q)), d.argmin(1)]
    assert np.allclose(outL, F[near], rtol=0, atol=1e-6)


def test_empty_rows_and_negative_scale():
    pts, q, F, dO, table = _small_case(N=3, K=5)
    slots, d, w = O.knn_weights(pts, q, table, -0.7)
    assert (slots[:, 3:] == -1).all() and (w[:, 3:] == 0).all()
    # negative p favours the farthest slot; still a normalised softmax
    assert np.allclose(w.sum(1), 1.0, atol=1e-14)
    assert (w[np.arange(len(q)), d[:, :3].argmax(1)] >= w[:, :3].max(1) - 1e-15).all()
    out = O.knn_sample_fwd(np.zeros((0, 2), np.float32), np.zeros((0, 5)), q,
                           O.knn_table(np.zeros((0, 2), np.float32), 8, 4), 1.0)
    assert np.array_equal(out, np.zeros((len(q), 5)))


@pytest.mark.parametrize("p", [1.3, -0.6, 0.0])
def test_gradients_match_finite_differences(p):
    pts, q, F, dO, table = _small_case()

    def loss(F_, q_, p_):
        return float((O.knn_sample_fwd(pts, F_, q_, table, p_) * dO).sum())

    dF, dq, dp = O.knn_sample_bwd(pts, F, q, table, p, dO)
    # features: the loss is linear in F
    h = 1e-3
    for (n, c) in [(0, 0), (3, 2), (7, 4), (11, 1), (19, 3)]:
        Fp, Fm = F.copy(), F.copy()
        Fp[n, c] += h
        Fm[n, c] -= h
        assert dF[n, c] == pytest.approx((loss(Fp, q, p) - loss(Fm, q, p)) / (2 * h), abs=1e-9)
    # query coordinates (f32): steps of 2**-10 are exact and stay inside the cell
    h = 2.0 ** -10
    for m in range(q.shape[0]):
        for a in range(2):
            qp, qm = q.copy(), q.copy()
            qp[m, a] += np.float32(h)
            qm[m, a] -= np.float32(h)
            fd = (loss(F, qp, p) - loss(F, qm, p)) / (2 * h)
            assert dq[m, a] == pytest.approx(fd, rel=1e-4, abs=1e-5), (m, a)
    h = 1e-6
    assert dp == pytest.approx((loss(F, q, p + h) - loss(F, q, p - h)) / (2 * h), rel=1e-6, abs=1e-8)


def test_zero_distance_gradient_is_zero():
    """A query on a token: that slot contributes nothing to dq (reading K7),
    and the other slots still do."""
    pts = np.array([[2, 2], [3, 2], [2, 4]], dtype=np.float32)
    q = np.array([[2, 2]], dtype=np.float32)
    table = O.knn_table(pts, 8, 3)
    F = np.eye(3)
    dO = np.array([[1.0, -2.0, 0.5]])
    dF, dq, dp = O.knn_sample_bwd(pts, F, q, table, 1.0, dO)
    assert np.all(np.isfinite(dq))
    _, d, w = O.knn_weights(pts, q, table, 1.0)
    g = dO[0]                                          # F = I: g_k = dO[token_k]
    slots = table[2, 2]
    gs = g[slots]
    ds = w[0] * (gs - (w[0] * gs).sum())
    units = [(q[0] - pts[t]) / max(np.hypot(*(q[0] - pts[t])), 1e-300) if t != 0 else np.zeros(2)
             for t in slots]
    expect = sum(-1.0 * ds[k] * units[k] for k in range(3))
    assert np.allclose(dq[0], expect, atol=1e-14)


def test_workload_generators_are_seeded():
    a = make_sampler_case("knn_tiny", tensors=True)
    b = make_sampler_case("knn_tiny", tensors=True)
    assert np.array_equal(a["queries"], b["queries"])
    for x, y in zip(a["feats"], b["feats"]):
        assert (x == y).all()
    dec = make_sampler_case("knn_decoder", B=1, tensors=False)
    assert [c.shape[1] for c in dec["coords"]] == [2048, 819, 328, 131]
    assert dec["queries"].shape == (1, 2048, 2)
