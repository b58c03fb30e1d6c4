"""Pins of the token-merging oracle (no GPU): hand-worked ties, an
independent threshold form of the top-k, a k-d tree check of the nearest
anchors, closed forms of the softmax merge and finite differences of every
gradient."""

import numpy as np
import pytest

import oracle as O
from gen import make_merge_case


def test_anchors_hand_worked_ties():
    s = np.array([0.5, 2.0, 0.5, -1.0, 2.0, 0.5], dtype=np.float32)
    # k = 3: both 2.0s, then the lowest-index 0.5 (token 0); listed ascending
    assert O.merge_anchors(s, 3).tolist() == [0, 1, 4]
    assert O.merge_anchors(s, 4).tolist() == [0, 1, 2, 4]
    assert O.merge_anchors(s, 6).tolist() == [0, 1, 2, 3, 4, 5]
    assert O.merge_anchors(s, 1).tolist() == [1]


def test_anchors_threshold_form():
    """The k-th largest value v: every token above v, and the lowest-index
    ones at v until k are taken."""
    rng = np.random.default_rng(1)
    for trial in range(20):
        N = int(rng.integers(1, 300))
        s = rng.integers(-5, 5, size=N).astype(np.float32)   # many ties
        k = int(rng.integers(1, N + 1))
        v = np.sort(s)[::-1][k - 1]
        above = np.nonzero(s > v)[0]
        at = np.nonzero(s == v)[0][: k - above.size]
        assert O.merge_anchors(s, k).tolist() == sorted(above.tolist() + at.tolist())


def test_assignment_hand_worked():
    # anchors at tokens 0 (0,0) and 2 (4,0); token 1 at (2,0) is equidistant:
    # the earlier anchor in the list wins; token 3 at (3,1) goes to anchor 2
    X = np.array([[0, 0], [2, 0], [4, 0], [3, 1]], dtype=np.float32)
    a = np.array([0, 2])
    assert O.merge_assign(X, a, 8).tolist() == [0, 0, 1, 1]


def test_assignment_matches_kdtree():
    from scipy.spatial import cKDTree

    rng = np.random.default_rng(2)
    G = 32
    X = rng.uniform(-0.5, G - 0.5, size=(400, 2)).astype(np.float32)
    X[300:] = X[:100]                                      # repeated coordinates
    s = rng.standard_normal(400).astype(np.float32)
    anchors = O.merge_anchors(s, 150)
    assign = O.merge_assign(X, anchors, G)
    qx, qy = O.quantize(X, G)
    P = np.stack([qx, qy], 1).astype(np.float64)
    tree = cKDTree(P[anchors])
    d, _ = tree.query(P, k=1)
    for i in range(400):
        if i in set(anchors.tolist()):
            assert anchors[assign[i]] == i
            continue
        d2 = ((P[anchors] - P[i]) ** 2).sum(1)
        assert d2[assign[i]] == round(d[i] ** 2)
        assert assign[i] == np.nonzero(d2 == d2.min())[0][0]


@pytest.mark.parametrize("geom,N,k,G", [("uniform", 500, 180, 32), ("dense", 256, 100, 16),
                                         ("dense", 1024, 410, 32), ("uniform", 50, 50, 8)])
def test_tree_assignment_matches_scan(geom, N, k, G):
    """The k-d tree form against the per-token scan: uniform points with
    repeated coordinates, and every cell of a dense grid (equidistant
    anchors everywhere), up to k = N."""
    rng = np.random.default_rng(N + k)
    if geom == "dense":
        cells = np.arange(G * G)[:N]
        X = np.stack([cells % G, cells // G], 1).astype(np.float32)
    else:
        X = rng.uniform(-0.5, G - 0.5, size=(N, 2)).astype(np.float32)
        X[N // 2:N // 2 + N // 5] = X[:N // 5]
    anchors = O.merge_anchors(rng.standard_normal(N).astype(np.float32), k)
    np.testing.assert_array_equal(O.merge_assign_tree(X, anchors, G), O.merge_assign(X, anchors, G))


def test_weights_match_per_group_softmax():
    """The gathered form of reading M4 against a softmax taken group by
    group (scipy's, on each group's scores)."""
    from scipy.special import softmax

    X, s, F, anchors, assign = _case(seed=9, N=120, k=30)
    w = O.merge_weights(s, assign, anchors.size)
    for a in range(anchors.size):
        g = assign == a
        np.testing.assert_allclose(w[g], softmax(s[g]), rtol=1e-14, atol=0)


def _case(seed=4, N=40, k=12, C=5):
    rng = np.random.default_rng(seed)
    X = rng.uniform(0, 10, size=(N, 2)).astype(np.float32)
    s = rng.standard_normal(N)
    F = rng.standard_normal((N, C))
    anchors = O.merge_anchors(s, k)
    assign = O.merge_assign(X, anchors, 16)
    return X, s, F, anchors, assign


def test_merge_closed_forms():
    X, s, F, anchors, assign = _case()
    k = anchors.size
    w = O.merge_weights(s, assign, k)
    sums = np.zeros(k)
    np.add.at(sums, assign, w)
    assert np.allclose(sums, 1.0, atol=1e-14)
    # equal scores: plain means
    Fm, Xm = O.merge_fwd(F, X, np.zeros_like(s), assign, k)
    for a in range(k):
        g = assign == a
        assert np.allclose(Fm[a], F[g].mean(0), atol=1e-14)
        assert np.allclose(Xm[a], X[g].astype(np.float64).mean(0), atol=1e-12)
    # singleton groups reproduce the anchor
    Fm, Xm = O.merge_fwd(F, X, s, assign, k)
    for a in range(k):
        g = np.nonzero(assign == a)[0]
        if g.size == 1:
            assert np.array_equal(Fm[a], F[g[0]])
        lo, hi = X[g].min(0), X[g].max(0)                 # inside the members' box
        assert (Xm[a] >= lo - 1e-12).all() and (Xm[a] <= hi + 1e-12).all()
    # a score shift common to a group changes nothing
    s2 = s + np.where(assign == 0, 3.0, 0.0)
    F2, X2 = O.merge_fwd(F, X, s2, assign, k)
    assert np.allclose(F2, Fm, atol=1e-13) and np.allclose(X2, Xm, atol=1e-12)


def test_merge_gradients_finite_differences():
    X, s, F, anchors, assign = _case()
    k = anchors.size
    rng = np.random.default_rng(9)
    dFm = rng.standard_normal((k, F.shape[1]))
    dXm = rng.standard_normal((k, 2))

    def loss(F_, X_, s_):
        Fm, Xm = O.merge_fwd(F_, X_, s_, assign, k)
        return float((Fm * dFm).sum() + (Xm * dXm).sum())

    dF, dX, ds = O.merge_bwd(F, X, s, assign, k, dFm, dXm)
    h = 1e-6
    for i in (0, 7, 19, 33):
        sp, sm = s.copy(), s.copy()
        sp[i] += h
        sm[i] -= h
        assert ds[i] == pytest.approx((loss(F, X, sp) - loss(F, X, sm)) / (2 * h), abs=1e-8)
        for c in (0, 3):
            Fp, Fmn = F.copy(), F.copy()
            Fp[i, c] += h
            Fmn[i, c] -= h
            assert dF[i, c] == pytest.approx((loss(Fp, X, s) - loss(Fmn, X, s)) / (2 * h), abs=1e-8)
    # coordinates are f32 inputs: the loss is linear in them, steps of 2^-8
    h = 2.0 ** -8
    for i in (1, 12, 30):
        for a in range(2):
            Xp, Xn = X.copy(), X.copy()
            Xp[i, a] += np.float32(h)
            Xn[i, a] -= np.float32(h)
            assert dX[i, a] == pytest.approx((loss(F, Xp, s) - loss(F, Xn, s)) / (2 * h), abs=1e-9)
    # sum rules: each group's dF adds up to dF'_a, its ds to 0
    for a in range(k):
        g = assign == a
        assert np.allclose(dF[g].sum(0), dFm[a], atol=1e-13)
        assert abs(ds[g].sum()) < 1e-12


def test_merge_workloads_are_seeded():
    a = make_merge_case("merge_tiny")
    b = make_merge_case("merge_tiny")
    assert all(np.array_equal(x, y) for x, y in zip(a["scores"], b["scores"]))
    st = make_merge_case("merge_stages", B=1, tensors=False)
    assert [c.shape[1] for c in st["coords"]] == [2048, 819, 328]
