"""Plain, slow, fp64 CPU oracle for the decoder's KNN-cache point sampler.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg, never by the product path.  It shares no code, header,
table or helper with the HIP library.

Source: the English notes page "AFFMAE: Scalable Vision Pre-Training for
High-Resolution Microscopy Segmentation on Desktop Hardware"
(en.papernotes.org), cited as [AFFMAE-notes]:

* "Key Designs" item 2 (point-wise deformable cross-attention decoder): a
  query predicts an offset and samples at q = r + offset; the nearest
  visible tokens around q are aggregated with weights w_i = softmax_i(-p d_i),
  the stable-softmax replacement of inverse-power weights d_i^(-p).
* "Key Designs" item 3 (KNN cache lookup): the token grid is a fixed
  H x W patch grid; an H x W x K table keeps, per grid cell, the indices of
  the K nearest visible tokens; a query is quantised to its nearest grid
  cell, so the search becomes a table lookup plus a distance calculation,
  and distance and softmax weighting are fused into one kernel (forward and
  backward).

The pages leave the distances, the cell rule and the gradients open.  The
readings taken here:

K1. the grid is the G x G token grid (H = W = G); cell (row i, column j) has
    its centre at (x, y) = (j, i) in patch units, where a token of the dense
    grid sits;
K2. a cell's K nearest tokens are ranked by the squared distance between
    the token's fixed-point coordinate (the 16-bit quantisation of the
    neighbour build, reading 1 of :mod:`oracle.cluster_attention`) and the
    cell centre in the same fixed point, ((j + 1/2) s, (i + 1/2) s), ties to
    the lower token index; -1 pads a row when the image has fewer than K
    tokens;
K3. a query (x, y) goes to the cell of the nearest centre,
    j = clamp(floor(x + 1/2), 0, G - 1) and likewise i from y (fp64 from the
    f32 inputs);
K4. d_k is the Euclidean distance between the query and the k-th token's
    f32 coordinate, in patch units;
K5. w = softmax over the valid slots of (-p d_k) for a real scalar p given
    by the caller (one per level), computed as the stable softmax;
K6. out = sum_k w_k F[token_k]; a query whose row has no valid slot gets 0;
K7. the backward returns the gradients with respect to F, to the query
    coordinates and to p; the token coordinates are constants; the
    derivative of d_k at d_k = 0 is taken as 0.

Everything is the plain definition: the table is a brute-force ranking,
the sampler the weighted sum, and the gradients the chain rule written out.
"""

from __future__ import annotations

import numpy as np

from .cluster_attention import quantize, grid_bits

__all__ = [
    "knn_table",
    "knn_table_cells",
    "query_cells",
    "knn_weights",
    "knn_sample_fwd",
    "knn_sample_bwd",
    "knn_table_batch",
    "knn_sample_fwd_batch",
    "knn_sample_bwd_batch",
]


def knn_table(coords: np.ndarray, grid_side: int, K: int) -> np.ndarray:
    """[AFFMAE-notes] "Key Designs" item 3, readings K1-K2, one image.

    coords [N, 2] float32 -> table [G, G, K] int64 (row i, column j)."""
    G = grid_side
    N = coords.shape[0]
    qx, qy = quantize(coords, G)                       # int64 fixed point
    s = 2 ** (16 - grid_bits(G))
    table = np.full((G, G, K), -1, dtype=np.int64)
    if N == 0:
        return table
    idx = np.arange(N, dtype=np.int64)
    take = min(K, N)
    for i in range(G):
        cy = (2 * i + 1) * s // 2                      # (i + 1/2) s, an integer
        for j in range(G):
            cx = (2 * j + 1) * s // 2
            d2 = (qx - cx) ** 2 + (qy - cy) ** 2       # exact int64
            order = np.lexsort((idx, d2))              # by d2, then index
            table[i, j, :take] = order[:take]
    return table


def knn_table_cells(coords: np.ndarray, grid_side: int, K: int, rows: np.ndarray,
                    cols: np.ndarray, chunk: int = 256) -> np.ndarray:
    """Readings K1-K2 for the listed cells only (row ``rows[c]``, column
    ``cols[c]``) of one image: [n, K] int64, equal to
    ``knn_table(coords, G, K)[rows, cols]``.

    For grids too large to rank every cell: each cell's tokens are ranked by
    the single integer d2 * 2^25 + index (d2 < 2^33 and index < 2^25, so it
    orders exactly as (d2, index)), the K smallest picked by a partial sort
    and then sorted."""
    G = grid_side
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    cols = np.asarray(cols, dtype=np.int64).reshape(-1)
    N = coords.shape[0]
    if N >= 2 ** 25:
        raise ValueError("token index must fit 25 bits")
    out = np.full((rows.size, K), -1, dtype=np.int64)
    if N == 0 or rows.size == 0:
        return out
    qx, qy = quantize(coords, G)
    s = 2 ** (16 - grid_bits(G))
    idx = np.arange(N, dtype=np.int64)
    take = min(K, N)
    for c0 in range(0, rows.size, chunk):
        cy = ((2 * rows[c0:c0 + chunk] + 1) * s // 2)[:, None]
        cx = ((2 * cols[c0:c0 + chunk] + 1) * s // 2)[:, None]
        key = ((qx[None, :] - cx) ** 2 + (qy[None, :] - cy) ** 2) * (2 ** 25) + idx[None, :]
        if take < N:
            part = np.partition(key, take - 1, axis=1)[:, :take]
        else:
            part = key
        part = np.sort(part, axis=1)[:, :take]
        out[c0:c0 + chunk, :take] = part % (2 ** 25)
    return out


def query_cells(queries: np.ndarray, grid_side: int) -> tuple[np.ndarray, np.ndarray]:
    """Reading K3: (row i, column j) of the nearest cell centre, int64."""
    q = np.asarray(queries)
    if q.dtype != np.float32:
        raise TypeError("queries must be float32")
    q64 = q.astype(np.float64)
    j = np.clip(np.floor(q64[..., 0] + 0.5), 0, grid_side - 1).astype(np.int64)
    i = np.clip(np.floor(q64[..., 1] + 0.5), 0, grid_side - 1).astype(np.int64)
    return i, j


def _rows(A: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """A[idx] (zeros when A has no rows; every index is then a padded slot)."""
    if A.shape[0] == 0:
        return np.zeros(idx.shape + A.shape[1:])
    return A[idx]


def knn_weights(coords, queries, table, p):
    """Readings K3-K5 for one image: slots [M, K] (-1 = empty), distances
    [M, K] (fp64, 0 on empty slots) and weights [M, K] (0 on empty slots)."""
    coords = np.asarray(coords, dtype=np.float32).astype(np.float64)
    G = table.shape[0]
    i, j = query_cells(queries, G)
    slots = table[i, j]                                # [M, K]
    q = np.asarray(queries, dtype=np.float32).astype(np.float64)
    valid = slots >= 0
    pos = _rows(coords, np.where(valid, slots, 0))     # [M, K, 2]
    diff = q[:, None, :] - pos
    d = np.sqrt((diff ** 2).sum(-1))
    d = np.where(valid, d, 0.0)
    logit = np.where(valid, -p * d, -np.inf)
    m = logit.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(valid, np.exp(logit - m), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    w = np.where(tot > 0, e / np.where(tot > 0, tot, 1.0), 0.0)
    return slots, d, w


def knn_sample_fwd(coords, feats, queries, table, p):
    """Reading K6 for one image: out [M, Cf] fp64."""
    F = np.asarray(feats, dtype=np.float64)
    slots, _, w = knn_weights(coords, queries, table, p)
    rows = _rows(F, np.where(slots >= 0, slots, 0))    # [M, K, Cf]
    return (w[:, :, None] * rows).sum(axis=1)


def knn_sample_bwd(coords, feats, queries, table, p, dout):
    """Reading K7 for one image: (dF [N, Cf], dq [M, 2], dp) in fp64.

    With g_k = <dout, F_k>, the softmax gives dL/ds_k = w_k (g_k - sum_j
    w_j g_j) for the logit s_k = -p d_k; then dL/dd_k = -p dL/ds_k,
    dd_k/dq = (q - x_k) / d_k (0 at d_k = 0), dL/dp = -sum_k dL/ds_k d_k,
    and dF[t] collects w_k dout over every (query, slot) that holds t."""
    F = np.asarray(feats, dtype=np.float64)
    dO = np.asarray(dout, dtype=np.float64)
    q = np.asarray(queries, dtype=np.float32).astype(np.float64)
    X = np.asarray(coords, dtype=np.float32).astype(np.float64)
    slots, d, w = knn_weights(coords, queries, table, p)
    valid = slots >= 0
    safe = np.where(valid, slots, 0)
    rows = _rows(F, safe)                              # [M, K, Cf]
    g = np.einsum("mc,mkc->mk", dO, rows)
    ds = w * (g - (w * g).sum(axis=1, keepdims=True))
    ds = np.where(valid, ds, 0.0)
    dd = -p * ds
    diff = q[:, None, :] - _rows(X, safe)
    unit = np.where((d > 0)[..., None], diff / np.where(d > 0, d, 1.0)[..., None], 0.0)
    dq = (dd[..., None] * unit).sum(axis=1)
    dp = float(-(ds * d).sum())
    dF = np.zeros_like(F)
    M, K = slots.shape
    for m in range(M):
        for k in range(K):
            if slots[m, k] >= 0:
                dF[slots[m, k]] += w[m, k] * dO[m]
    return dF, dq, dp


# ---- batches: images are independent ---------------------------------------

def knn_table_batch(coords: np.ndarray, grid_side: int, K: int) -> np.ndarray:
    """coords [B, N, 2] float32 -> [B, G, G, K] int32."""
    return np.stack([knn_table(c, grid_side, K) for c in coords]).astype(np.int32)


def knn_sample_fwd_batch(coords, feats, queries, table, p):
    return np.stack([knn_sample_fwd(coords[b], feats[b], queries[b], table[b], p)
                     for b in range(len(coords))])


def knn_sample_bwd_batch(coords, feats, queries, table, p, dout):
    res = [knn_sample_bwd(coords[b], feats[b], queries[b], table[b], p, dout[b])
           for b in range(len(coords))]
    dF = np.stack([r[0] for r in res])
    dq = np.stack([r[1] for r in res])
    dp = float(sum(r[2] for r in res))
    return dF, dq, dp
