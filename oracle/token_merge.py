"""Plain, slow, fp64 CPU oracle for adaptive off-grid token merging.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg, never by the product path.  It shares no code, header,
table or helper with the HIP library.

Source: the English notes page "AFFMAE: Scalable Vision Pre-Training for
High-Resolution Microscopy Segmentation on Desktop Hardware"
(en.papernotes.org), "Key Designs" item 1 (adaptive off-grid token
merging), cited as [AFFMAE-notes]: every token carries its 2D coordinate; a
lightweight MLP scores the tokens, the top-k by the retention rate are kept
as anchors, and the other tokens are merged, differentiably, into their
nearest anchors, features and spatial support alike; "A Complete Example"
gives the retention rate 0.4 (2048 -> 819 -> 328 -> 131 tokens).

The pages leave the scores, the distance, the ties and the merge weights
open.  Readings (M1-M7):

M1. the scores are an input (the MLP that makes them is not part of this
    op); k is given by the caller (round(0.4 N) in the workloads);
M2. anchors: the k tokens with the largest scores, ties to the lower token
    index, listed in ascending token index (merged tokens keep the image's
    order);
M3. every anchor is assigned to itself; every other token to the anchor
    whose fixed-point coordinate (the 16-bit quantisation of the neighbour
    build, reading 1 of :mod:`oracle.cluster_attention`) is nearest by
    squared distance, ties to the anchor earlier in the list;
M4. "differentiably merged": within an anchor's group G_a the weights are
    the softmax of the members' scores, w_i = exp(s_i) / sum_{j in G_a}
    exp(s_j) (so that the scores receive gradients);
M5. merged feature F'_a = sum_i w_i F_i and merged coordinate
    X'_a = sum_i w_i X_i (the spatial support is merged like the features);
M6. the backward returns the gradients with respect to F, X and s, with the
    anchors and the assignment held fixed (they are discrete);
M7. fp64 here; the kernels accumulate in fp32.
"""

from __future__ import annotations

import numpy as np

from .cluster_attention import quantize

__all__ = [
    "merge_anchors",
    "merge_assign",
    "merge_assign_tree",
    "merge_weights",
    "merge_fwd",
    "merge_bwd",
]


def merge_anchors(scores: np.ndarray, k: int) -> np.ndarray:
    """Reading M2 for one image: the anchor token indices, ascending, int64."""
    s = np.asarray(scores, dtype=np.float64)
    N = s.shape[0]
    k = min(k, N)
    idx = np.arange(N, dtype=np.int64)
    order = np.lexsort((idx, -s))          # by score descending, then index
    return np.sort(order[:k])


def merge_assign(coords: np.ndarray, anchors: np.ndarray, grid_side: int) -> np.ndarray:
    """Reading M3 for one image: assign[i] = position in `anchors` of the
    anchor of token i (int64)."""
    qx, qy = quantize(np.asarray(coords, dtype=np.float32), grid_side)
    N = qx.shape[0]
    k = anchors.shape[0]
    assign = np.empty(N, dtype=np.int64)
    pos = np.arange(k, dtype=np.int64)
    for i in range(N):
        d2 = (qx[anchors] - qx[i]) ** 2 + (qy[anchors] - qy[i]) ** 2
        assign[i] = np.lexsort((pos, d2))[0]
    assign[anchors] = pos                  # anchors anchor themselves
    return assign


def merge_assign_tree(coords: np.ndarray, anchors: np.ndarray, grid_side: int) -> np.ndarray:
    """Reading M3 for images too large for the per-token scan of
    :func:`merge_assign`; the same result.

    A k-d tree over the anchors' fixed-point coordinates (integers, exact in
    fp64) gives every token's nearest distance and then every anchor within
    a hair above it; among those, the exact integer squared distances pick
    the nearest, ties to the earlier anchor."""
    from scipy.spatial import cKDTree

    qx, qy = quantize(np.asarray(coords, dtype=np.float32), grid_side)
    P = np.stack([qx, qy], 1)
    A = P[anchors]
    tree = cKDTree(A.astype(np.float64))
    dmin, _ = tree.query(P.astype(np.float64), k=1)
    near = tree.query_ball_point(P.astype(np.float64), dmin * (1 + 1e-9) + 1e-6)
    assign = np.empty(P.shape[0], dtype=np.int64)
    for i, cand in enumerate(near):
        c = np.asarray(cand, dtype=np.int64)
        d2 = ((A[c] - P[i]) ** 2).sum(1)
        assign[i] = c[d2 == d2.min()].min()
    assign[anchors] = np.arange(anchors.shape[0], dtype=np.int64)
    return assign


def merge_weights(scores: np.ndarray, assign: np.ndarray, k: int) -> np.ndarray:
    """Reading M4: softmax of the scores inside every group (fp64), with the
    group maxima and sums gathered by group index."""
    s = np.asarray(scores, dtype=np.float64)
    a = np.asarray(assign, dtype=np.int64)
    gmax = np.full(k, -np.inf)
    np.maximum.at(gmax, a, s)
    e = np.exp(s - gmax[a])
    tot = np.bincount(a, weights=e, minlength=k)
    return e / tot[a]


def merge_fwd(feats, coords, scores, assign, k):
    """Reading M5 for one image: (F' [k, C], X' [k, 2]) in fp64."""
    F = np.asarray(feats, dtype=np.float64)
    X = np.asarray(coords, dtype=np.float32).astype(np.float64)
    w = merge_weights(scores, assign, k)
    Fm = np.zeros((k, F.shape[1]))
    Xm = np.zeros((k, 2))
    np.add.at(Fm, assign, w[:, None] * F)
    np.add.at(Xm, assign, w[:, None] * X)
    return Fm, Xm


def merge_bwd(feats, coords, scores, assign, k, dFm, dXm):
    """Reading M6 for one image: (dF [N, C], dX [N, 2], ds [N]) in fp64.

    With g_i = <dF'_a, F_i> + <dX'_a, X_i> for the group a of token i, the
    softmax gives ds_i = w_i (g_i - sum_{j in G_a} w_j g_j); dF_i = w_i dF'_a
    and dX_i = w_i dX'_a."""
    F = np.asarray(feats, dtype=np.float64)
    X = np.asarray(coords, dtype=np.float32).astype(np.float64)
    dFm = np.asarray(dFm, dtype=np.float64)
    dXm = np.asarray(dXm, dtype=np.float64)
    w = merge_weights(scores, assign, k)
    g = (dFm[assign] * F).sum(1) + (dXm[assign] * X).sum(1)
    gbar = np.zeros(k)
    np.add.at(gbar, assign, w * g)
    ds = w * (g - gbar[assign])
    return w[:, None] * dFm[assign], w[:, None] * dXm[assign], ds
