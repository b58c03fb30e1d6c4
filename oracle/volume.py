"""Plain CPU oracle of the neighbour build for 3D (volumetric) tokens.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg, never by the product path.  It shares no code,
header, table or helper with the HIP library.

Source: the English notes page "AFFMAE: Scalable Vision Pre-Training for
High-Resolution Microscopy Segmentation on Desktop Hardware", "Limitations &
Future Work": the paper sees no fundamental architectural barrier to 3D
voxels, and names cluster balancing and neighbourhood lookup in 3D as open.
The pages give no 3D algorithm; the readings here carry the 2D ones of
:mod:`oracle.cluster_attention` over to three axes:

V1. coordinates are (x, y, z) = (column, row, slice) in patch units on a
    grid of side G (the largest side of the volume's patch grid);
V2. each axis is quantised to 14-bit fixed point,
    q = clamp(floor((c + 1/2) * 2**(14 - ceil(log2 G))), 0, 2**14 - 1), in
    fp64 from the f32 inputs (14 bits per axis keep the 42-bit code and a
    22-bit token index in one 64-bit sort key);
V3. the Morton code interleaves the axes bit by bit: bit b of qx goes to bit
    3b, of qy to 3b + 1, of qz to 3b + 2;
V4. clusters, centroids (means, exact with the 840/n scaling), neighbour
    selection by (squared centroid distance, index), key lists and ragged or
    packed batches are exactly the 2D readings 3, 4 and 7, with three
    coordinates per centroid.

The attention itself does not depend on the dimension: the same oracle
functions (and the same kernels) consume the 3D lists.
"""

from __future__ import annotations

import numpy as np

from .cluster_attention import (balanced_clusters, centroid_keys, cluster_rows, grid_bits,
                                key_lists, nearest_clusters)

__all__ = ["quantize3", "morton_code3", "build_image3", "build_neighbors_3d",
           "build_neighbors_varlen_3d"]

BITS = 14


def quantize3(coords: np.ndarray, grid_side: int):
    """Reading V2: (qx, qy, qz) int64 from coords [..., 3] float32."""
    c = np.asarray(coords)
    if c.dtype != np.float32:
        raise TypeError("coords must be float32")
    step = float(2 ** (BITS - grid_bits(grid_side)))
    q = np.floor((c.astype(np.float64) + 0.5) * step)
    q = np.clip(q, 0.0, float(2 ** BITS - 1)).astype(np.int64)
    return q[..., 0], q[..., 1], q[..., 2]


def morton_code3(qx, qy, qz) -> np.ndarray:
    """Reading V3: 42-bit Z-order code, int64."""
    qx, qy, qz = (np.asarray(a, dtype=np.int64) for a in (qx, qy, qz))
    code = np.zeros(np.broadcast(qx, qy, qz).shape, dtype=np.int64)
    for b in range(BITS):
        code |= ((qx >> b) & 1) << (3 * b)
        code |= ((qy >> b) & 1) << (3 * b + 1)
        code |= ((qz >> b) & 1) << (3 * b + 2)
    return code


def build_image3(coords: np.ndarray, grid_side: int, cs: int = 8, k: int = 6):
    """Readings V1-V4 for one volume of any size N >= 0: q_idx [C, cs],
    nbr [C, k], key_idx [C, k*cs] (int64, image-local ids, -1 padding)."""
    qx, qy, qz = quantize3(np.asarray(coords), grid_side)
    q_idx = cluster_rows(balanced_clusters(morton_code3(qx, qy, qz)), cs)
    S = centroid_keys(q_idx, qx, qy, qz, cs=cs)
    nbr = nearest_clusters(S, k)
    _, key_idx = key_lists(q_idx, nbr, cs)
    return q_idx, nbr, key_idx


def build_neighbors_3d(coords: np.ndarray, grid_side: int, cs: int = 8, k: int = 6):
    """coords [B, N, 3] float32 -> perm [B, C*cs] (q_idx rows), nbr
    [B, C, k], key_idx [B, C, k*cs], int32, image-local."""
    coords = np.asarray(coords)
    B, N, three = coords.shape
    assert three == 3
    C = -(-N // cs)
    perm = np.empty((B, C * cs), dtype=np.int32)
    nbr = np.empty((B, C, k), dtype=np.int32)
    key_idx = np.empty((B, C, k * cs), dtype=np.int32)
    for b in range(B):
        qi, nb, kl = build_image3(coords[b], grid_side, cs, k)
        perm[b], nbr[b], key_idx[b] = qi.reshape(-1), nb, kl
    return perm, nbr, key_idx


def build_neighbors_varlen_3d(coords: np.ndarray, lengths, grid_side: int, cs: int = 8, k: int = 6):
    """Packed volumes (coords [T, 3]): as the 2D packed build, batch-global
    ids.  Returns q_idx, nbr, key_idx (int32), tok_off, clu_off."""
    lengths = [int(n) for n in lengths]
    tok_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    clu_off = np.concatenate([[0], np.cumsum([-(-n // cs) for n in lengths])]).astype(np.int64)
    qs, ns, ks = [], [], []
    for b, n in enumerate(lengths):
        qi, nb, kl = build_image3(np.asarray(coords)[tok_off[b]:tok_off[b + 1]], grid_side, cs, k)
        qs.append(np.where(qi >= 0, qi + tok_off[b], -1))
        ns.append(np.where(nb >= 0, nb + clu_off[b], -1))
        ks.append(np.where(kl >= 0, kl + tok_off[b], -1))
    cat = lambda xs, w: (np.concatenate(xs) if xs else np.zeros((0, w), np.int64)).astype(np.int32)
    return cat(qs, cs), cat(ns, k), cat(ks, k * cs), tok_off, clu_off
