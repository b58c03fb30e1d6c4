"""Plain, slow, fp64 CPU oracle for local cluster attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.  It shares
no code, header, table or helper with the HIP library.

Sources.  The method is described on the English notes page "AFFMAE: Scalable
Vision Pre-Training for High-Resolution Microscopy Segmentation on Desktop
Hardware" (en.papernotes.org, ECCV2026), cited below as [AFFMAE-notes], and in
the arXiv abstract reproduced on the mlsanity.com page of the same title,
cited as [AFFMAE-abs].

* [AFFMAE-notes] "Overall Architecture": every token keeps an explicit 2D
  coordinate and attention is computed through local balanced clustering.
* [AFFMAE-abs] and [AFFMAE-notes] "Background & Motivation": the attention
  runs in numerically stable, mixed-precision, Flash-style kernels.
* [AFFMAE-notes] "Limitations & Future Work": off-grid gather/scatter is what
  costs time; space-filling curves are named as the lookup structure.

The pages leave the clustering, the neighbourhood rule, the scale and the
precision open.  The readings taken here (all listed in the design doc):

1. coordinates are quantised to 16-bit fixed point per axis with
   ``2**(16 - ceil(log2 G))`` steps per grid unit, G the grid side;
2. the space-filling curve is the Morton (Z) order with x in the even bits;
3. "balanced clusters" are consecutive runs of ``cs`` tokens in that order,
   ties in the code broken by token index (a stable sort);
4. each cluster attends to itself plus the ``k-1`` clusters whose integer
   centroid sums are nearest (squared distance, ties by lower cluster index);
5. attention is plain scaled-dot-product softmax attention restricted to the
   gathered key slots, scale supplied by the caller (1/sqrt(D) in every
   workload), a repeated slot counting with multiplicity, slot -1 masked;
6. LSE is the natural log-sum-exp of the scaled logits;
7. ragged images: when N is not a multiple of cs the last run of the order
   is one partial cluster of n = N - cs*(C-1) members (C = ceil(N/cs)); its
   q_idx row, and every key slot standing for an absent member, is -1.
   Clusters are compared through their centroids (means), written as exact
   integers by scaling every coordinate sum by L/n with L = lcm(1..cs)
   (840 for cs = 8), which for full clusters is a constant factor and so
   leaves the full-cluster order unchanged.  Images of different sizes are
   packed one after another (per-image token and cluster offsets) and then
   use batch-global token and cluster ids.

Forward and backward are exact softmax attention, so the oracle writes the
plain definition (a count-masked dense form and an equivalent per-cluster
gathered form).  The neighbour build is a heuristic and is written as its
steps, in order.  All floating point is fp64; integer steps are exact.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "quantize",
    "morton_code",
    "balanced_clusters",
    "centroid_sums",
    "cluster_rows",
    "centroid_keys",
    "nearest_clusters",
    "nearest_clusters_fullsort",
    "key_lists",
    "build_neighbors",
    "build_image",
    "build_neighbors_varlen",
    "count_matrix",
    "attn_fwd_dense",
    "attn_fwd_gathered",
    "attn_bwd_dense",
    "attn_bwd_gathered",
]


# ---------------------------------------------------------------------------
# Neighbour-list build: [AFFMAE-notes] "Overall Architecture" (2D coordinate
# per token, local balanced clustering) and "Limitations & Future Work"
# (space-filling curves).  Readings 1-4 of the module docstring.
# ---------------------------------------------------------------------------

def grid_bits(grid_side: int) -> int:
    """ceil(log2(G)) for an integer grid side G >= 1."""
    if grid_side < 1 or grid_side > 65536:
        raise ValueError("grid side must be in [1, 65536]")
    return int(grid_side - 1).bit_length()


def quantize(coords: np.ndarray, grid_side: int) -> tuple[np.ndarray, np.ndarray]:
    """Fixed-point coordinates (reading 1).

    ``coords[..., 0]`` is x (column), ``coords[..., 1]`` is y (row), in patch
    units.  q = clamp(floor((c + 0.5) * 2**(16 - ceil(log2 G))), 0, 65535),
    evaluated in fp64 from the f32 inputs.  Returns (qx, qy) as int64.
    """
    c = np.asarray(coords)
    if c.dtype != np.float32:
        raise TypeError("coords must be float32")
    shift = 16 - grid_bits(grid_side)
    step = float(2 ** shift)
    c64 = c.astype(np.float64)
    q = np.floor((c64 + 0.5) * step)
    q = np.clip(q, 0.0, 65535.0).astype(np.int64)
    return q[..., 0], q[..., 1]


def morton_code(qx: np.ndarray, qy: np.ndarray) -> np.ndarray:
    """Z-order code of 16-bit (qx, qy): bit b of qx goes to bit 2b, bit b of
    qy to bit 2b+1 (reading 2).  Returns int64 in [0, 2**32)."""
    qx = np.asarray(qx, dtype=np.int64)
    qy = np.asarray(qy, dtype=np.int64)
    code = np.zeros(np.broadcast(qx, qy).shape, dtype=np.int64)
    for b in range(16):
        code |= ((qx >> b) & 1) << (2 * b)
        code |= ((qy >> b) & 1) << (2 * b + 1)
    return code


def balanced_clusters(code: np.ndarray) -> np.ndarray:
    """Stable sort of one image's tokens by (code, token index) (reading 3).

    Returns ``perm`` (int64, length N); cluster c is perm[c*cs:(c+1)*cs].
    """
    code = np.asarray(code, dtype=np.int64)
    idx = np.arange(code.shape[0], dtype=np.int64)
    # np.lexsort sorts by the last key first: primary = code, secondary = index
    return np.lexsort((idx, code))


def centroid_sums(perm: np.ndarray, qx: np.ndarray, qy: np.ndarray, cs: int) -> np.ndarray:
    """Integer sums of the members' fixed-point coordinates, [C, 2] int64.

    Every cluster has exactly cs members, so comparing sums compares means."""
    members = perm.reshape(-1, cs)
    return np.stack([qx[members].sum(axis=1), qy[members].sum(axis=1)], axis=1)


def cluster_rows(perm: np.ndarray, cs: int) -> np.ndarray:
    """Reading 7: the order cut into runs of cs, the last run padded with -1.
    Returns q_idx [ceil(N/cs), cs] int64."""
    perm = np.asarray(perm, dtype=np.int64)
    N = perm.shape[0]
    C = -(-N // cs)
    rows = np.full(C * cs, -1, dtype=np.int64)
    rows[:N] = perm
    return rows.reshape(C, cs)


def centroid_keys(q_idx: np.ndarray, *axes, cs: int = 8) -> np.ndarray:
    """Reading 7: every cluster's mean fixed-point coordinate times
    L = lcm(1..cs), as exact integers: (sum of the n members) * (L / n),
    one column per axis (qx, qy[, qz]).  [C, len(axes)] int64 (below 2**26
    for cs = 8, so squared distances fit int64)."""
    L = math.lcm(*range(1, cs + 1))
    live = q_idx >= 0
    safe = np.where(live, q_idx, 0)
    n = live.sum(axis=1)                      # members per cluster, >= 1
    cols = [np.where(live, np.asarray(a)[safe], 0).sum(axis=1) * (L // n) for a in axes]
    return np.stack(cols, axis=1).astype(np.int64)


def _sq_dist(S: np.ndarray, rows: np.ndarray) -> np.ndarray:
    d2 = np.zeros((rows.size, S.shape[0]), dtype=np.int64)
    for a in range(S.shape[1]):              # every axis of the centroids
        d = S[rows, a][:, None] - S[None, :, a]
        d2 += d * d
    return d2  # exact int64 (scaled sums below 2**26)


def nearest_clusters(S: np.ndarray, k: int, block: int = 512) -> np.ndarray:
    """Reading 4: slot 0 = self, then the k-1 other clusters with the smallest
    (squared centroid distance, cluster index), ascending; -1 pads when
    the image has fewer than k clusters.  Returns [C, k] int64.

    Brute force over all clusters of the image: every cluster whose distance
    is at most the (k-1)-th smallest is a candidate (ties included), and the
    candidates, listed by index, are sorted stably by distance."""
    C = S.shape[0]
    out = np.full((C, k), -1, dtype=np.int64)
    out[:, 0] = np.arange(C)
    take = min(k - 1, C - 1)
    if take <= 0:
        return out
    for r0 in range(0, C, block):
        rows = np.arange(r0, min(C, r0 + block))
        d2 = _sq_dist(S, rows)
        d2[np.arange(rows.size), rows] = np.iinfo(np.int64).max  # exclude self
        kth = np.partition(d2, take - 1, axis=1)[:, take - 1]
        for i, r in enumerate(rows):
            cand = np.nonzero(d2[i] <= kth[i])[0]
            order = cand[np.argsort(d2[i, cand], kind="stable")]
            out[r, 1:1 + take] = order[:take]
    return out


def nearest_clusters_fullsort(S: np.ndarray, k: int) -> np.ndarray:
    """Second formulation of reading 4 (used as a cross-check): a full
    lexicographic sort of all candidates of every cluster by (d2, index)."""
    C = S.shape[0]
    out = np.full((C, k), -1, dtype=np.int64)
    for c in range(C):
        d2 = ((S - S[c]) ** 2).sum(axis=1)
        cand = np.array([b for b in range(C) if b != c], dtype=np.int64)
        order = cand[np.lexsort((cand, d2[cand]))]
        row = [c] + list(order[: k - 1])
        out[c, : len(row)] = row
    return out


def key_lists(perm: np.ndarray, nbr: np.ndarray, cs: int) -> tuple[np.ndarray, np.ndarray]:
    """q_idx[c, m] = perm[c*cs + m] (-1 past the end of the order);
    key_idx[c, s*cs + m] = q_idx[nbr[c,s], m] (or -1 where nbr is -1).
    ``perm`` may be given as the order [N] or as q_idx rows [C, cs].
    Returns int64 arrays [C, cs] and [C, k*cs]."""
    C, k = nbr.shape
    perm = np.asarray(perm, dtype=np.int64)
    q_idx = perm if perm.ndim == 2 else cluster_rows(perm, cs)
    key_idx = np.full((C, k * cs), -1, dtype=np.int64)
    for s in range(k):
        valid = nbr[:, s] >= 0
        key_idx[valid, s * cs:(s + 1) * cs] = q_idx[nbr[valid, s]]
    return q_idx, key_idx


def build_image(coords: np.ndarray, grid_side: int, cs: int = 8, k: int = 6):
    """Readings 1-4 and 7 for one image of any size N >= 0: returns q_idx
    [C, cs], nbr [C, k] and key_idx [C, k*cs] (int64, image-local ids,
    C = ceil(N/cs), -1 padding)."""
    coords = np.asarray(coords)
    qx, qy = quantize(coords, grid_side)
    perm = balanced_clusters(morton_code(qx, qy))
    q_idx = cluster_rows(perm, cs)
    S = centroid_keys(q_idx, qx, qy, cs=cs)
    nbr = nearest_clusters(S, k)
    _, key_idx = key_lists(q_idx, nbr, cs)
    return q_idx, nbr, key_idx


def build_neighbors(coords: np.ndarray, grid_side: int, cs: int = 8, k: int = 6):
    """Whole neighbour build for a batch of equal-size images.

    coords [B, N, 2] float32  ->  perm [B, C*cs] (the q_idx rows [B, C, cs]
    flattened; equal to the token order when cs divides N, -1 padded
    otherwise), nbr [B, C, k], key_idx [B, C, k*cs], all int32 and
    image-local, C = ceil(N/cs)."""
    coords = np.asarray(coords)
    B, N, two = coords.shape
    assert two == 2
    C = -(-N // cs)
    perm = np.empty((B, C * cs), dtype=np.int32)
    nbr = np.empty((B, C, k), dtype=np.int32)
    key_idx = np.empty((B, C, k * cs), dtype=np.int32)
    for b in range(B):
        qi, nb, kl = build_image(coords[b], grid_side, cs, k)
        perm[b] = qi.reshape(-1)
        nbr[b] = nb
        key_idx[b] = kl
    return perm, nbr, key_idx


def build_neighbors_varlen(coords: np.ndarray, lengths, grid_side: int, cs: int = 8, k: int = 6):
    """Reading 7, packed batch: coords [T, 2] float32 holds the images one
    after another, image b having lengths[b] tokens.  Every image is built
    on its own; the results are concatenated with batch-global ids (token
    ids offset by the image's first token, cluster ids by its first
    cluster).  Returns q_idx [Ct, cs], nbr [Ct, k], key_idx [Ct, k*cs]
    (int32, -1 padding), tok_off [B+1] and clu_off [B+1] (int64)."""
    coords = np.asarray(coords)
    lengths = [int(n) for n in lengths]
    tok_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    clu_off = np.concatenate([[0], np.cumsum([-(-n // cs) for n in lengths])]).astype(np.int64)
    qs, ns, ks = [], [], []
    for b, n in enumerate(lengths):
        qi, nb, kl = build_image(coords[tok_off[b]:tok_off[b + 1]], grid_side, cs, k)
        qs.append(np.where(qi >= 0, qi + tok_off[b], -1))
        ns.append(np.where(nb >= 0, nb + clu_off[b], -1))
        ks.append(np.where(kl >= 0, kl + tok_off[b], -1))
    cat = lambda xs, w: (np.concatenate(xs) if xs else np.zeros((0, w), np.int64)).astype(np.int32)
    return cat(qs, cs), cat(ns, k), cat(ks, k * cs), tok_off, clu_off


# ---------------------------------------------------------------------------
# Attention: exact masked softmax attention restricted to the gathered slots
# ([AFFMAE-notes] "Overall Architecture": local cluster attention blocks;
# [AFFMAE-abs]: Flash-style kernels, whose result is exact attention).
# Reading 5 (slots with multiplicity, -1 masked) and reading 6 (natural LSE).
# ---------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: promote exactly through float64
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def count_matrix(q_idx: np.ndarray, key_idx: np.ndarray, N: int) -> np.ndarray:
    """M[i, j] = number of slots in the list of token i's cluster equal to j.

    q_idx [C, cs] and key_idx [C, nk] for one image.  Tokens that are in no
    cluster get an all-zero row."""
    M = np.zeros((N, N), dtype=np.float64)
    for c in range(q_idx.shape[0]):
        row = np.zeros(N, dtype=np.float64)
        for j in key_idx[c]:
            if j >= 0:
                row[j] += 1.0
        for i in q_idx[c]:
            if i >= 0:                      # -1: absent member of a partial cluster
                M[i] = row
    return M


def attn_fwd_dense(q, k, v, q_idx, key_idx, scale):
    """Definition form (count-masked dense attention), per image and head.

    S = scale * Q K^T; m_i = max over {j : M_ij > 0} of S_ij;
    Z_i = sum_j M_ij exp(S_ij - m_i); O_i = sum_j M_ij exp(S_ij - m_i) V_j / Z_i;
    LSE_i = m_i + ln Z_i.  A row with no valid slot gives O = 0, LSE = -inf.

    q, k, v [B, N, H, D]; q_idx [B, C, cs]; key_idx [B, C, nk].
    Returns O [B, N, H, D] and LSE [B, N, H], fp64."""
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, N, H, D = Q.shape
    O = np.zeros((B, N, H, D))
    LSE = np.full((B, N, H), -np.inf)
    for b in range(B):
        M = count_matrix(np.asarray(q_idx[b]), np.asarray(key_idx[b]), N)
        valid = M > 0
        has = valid.any(axis=1)
        for h in range(H):
            S = scale * (Q[b, :, h, :] @ K[b, :, h, :].T)
            Sm = np.where(valid, S, -np.inf)
            m = Sm.max(axis=1)
            m = np.where(has, m, 0.0)
            E = M * np.exp(np.where(valid, S - m[:, None], -np.inf))
            Z = E.sum(axis=1)
            Zs = np.where(has, Z, 1.0)
            P = E / Zs[:, None]
            O[b, :, h, :] = P @ V[b, :, h, :]
            LSE[b, :, h] = np.where(has, m + np.log(Zs), -np.inf)
    return O, LSE


def _gather_rows(X: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """X[idx] with -1 entries replaced by zero rows."""
    safe = np.where(idx >= 0, idx, 0)
    G = X[safe]
    G[idx < 0] = 0.0
    return G


def attn_fwd_gathered(q, k, v, q_idx, key_idx, scale, cluster_block: int = 1024):
    """Gathered form: the same definition evaluated on each cluster's
    cs x nk tile of gathered keys (slot -1 -> logit -inf).  Equal to
    :func:`attn_fwd_dense` up to fp64 rounding; needed where N*N is too large."""
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, N, H, D = Q.shape
    O = np.zeros((B, N, H, D))
    LSE = np.full((B, N, H), -np.inf)
    for b in range(B):
        qi = np.asarray(q_idx[b]).astype(np.int64)
        ki = np.asarray(key_idx[b]).astype(np.int64)
        C = qi.shape[0]
        for c0 in range(0, C, cluster_block):
            qb, kb = qi[c0:c0 + cluster_block], ki[c0:c0 + cluster_block]
            Qc = _gather_rows(Q[b], qb)        # [c, cs, H, D]; absent members: 0
            Kg = _gather_rows(K[b], kb)        # [c, nk, H, D]
            Vg = _gather_rows(V[b], kb)
            S = scale * np.einsum("cmhd,cshd->chms", Qc, Kg)
            valid = (kb >= 0)[:, None, None, :]
            has = valid.any(axis=-1)           # [c, 1, 1]
            m = np.where(valid, S, -np.inf).max(axis=-1)
            m = np.where(has, m, 0.0)
            E = np.where(valid, np.exp(S - m[..., None]), 0.0)
            Z = E.sum(axis=-1)
            Zs = np.where(has, Z, 1.0)
            P = E / Zs[..., None]
            Oc = np.einsum("chms,cshd->cmhd", P, Vg)
            L = np.where(has, m + np.log(Zs), -np.inf)   # [c, H, cs]
            live = qb >= 0                     # absent members write nothing
            O[b][qb[live]] = Oc[live]
            LSE[b][qb[live]] = np.transpose(L, (0, 2, 1))[live]
    return O, LSE


def attn_bwd_dense(q, k, v, do, q_idx, key_idx, scale):
    """Gradients of L = sum(dO * O) with the index lists held constant.

    With P the normalised, multiplicity-weighted probabilities of the
    forward: Delta_i = sum_d dO_id O_id; dP = dO V^T; dS = P * (dP - Delta);
    dQ = scale dS K; dK = scale dS^T Q; dV = P^T dO.
    Returns dQ, dK, dV [B, N, H, D] fp64."""
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, H, D = Q.shape
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        M = count_matrix(np.asarray(q_idx[b]), np.asarray(key_idx[b]), N)
        valid = M > 0
        has = valid.any(axis=1)
        for h in range(H):
            S = scale * (Q[b, :, h, :] @ K[b, :, h, :].T)
            m = np.where(has, np.where(valid, S, -np.inf).max(axis=1), 0.0)
            E = M * np.exp(np.where(valid, S - m[:, None], -np.inf))
            Z = np.where(has, E.sum(axis=1), 1.0)
            P = E / Z[:, None]
            Oh = P @ V[b, :, h, :]
            dOh = dO[b, :, h, :]
            delta = (dOh * Oh).sum(axis=1)
            dP = dOh @ V[b, :, h, :].T
            dS = P * (dP - delta[:, None])
            dQ[b, :, h, :] = scale * (dS @ K[b, :, h, :])
            dK[b, :, h, :] = scale * (dS.T @ Q[b, :, h, :])
            dV[b, :, h, :] = P.T @ dOh
    return dQ, dK, dV


def attn_bwd_gathered(q, k, v, do, q_idx, key_idx, scale, cluster_block: int = 1024):
    """Gathered form of :func:`attn_bwd_dense`: per cluster tile, with the
    dK/dV contributions of every slot accumulated by ``np.add.at`` (so a
    repeated slot adds twice and slot -1 adds nothing)."""
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, H, D = Q.shape
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        qi = np.asarray(q_idx[b]).astype(np.int64)
        ki = np.asarray(key_idx[b]).astype(np.int64)
        C = qi.shape[0]
        for c0 in range(0, C, cluster_block):
            qb, kb = qi[c0:c0 + cluster_block], ki[c0:c0 + cluster_block]
            Qc, dOc = _gather_rows(Q[b], qb), _gather_rows(dO[b], qb)   # [c, cs, H, D]
            Kg = _gather_rows(K[b], kb)            # [c, nk, H, D]
            Vg = _gather_rows(V[b], kb)
            S = scale * np.einsum("cmhd,cshd->chms", Qc, Kg)
            valid = (kb >= 0)[:, None, None, :]
            has = valid.any(axis=-1)
            m = np.where(has, np.where(valid, S, -np.inf).max(axis=-1), 0.0)
            E = np.where(valid, np.exp(S - m[..., None]), 0.0)
            Z = np.where(has, E.sum(axis=-1), 1.0)
            P = E / Z[..., None]                   # [c, H, cs, nk]
            P = P * (qb >= 0)[:, None, :, None]    # absent members: no query
            Oc = np.einsum("chms,cshd->cmhd", P, Vg)
            delta = np.einsum("cmhd,cmhd->chm", dOc, Oc)
            dP = np.einsum("cmhd,cshd->chms", dOc, Vg)
            dS = P * (dP - delta[..., None])
            live = qb >= 0
            dQ[b][qb[live]] = scale * np.einsum("chms,cshd->cmhd", dS, Kg)[live]
            dKg = scale * np.einsum("chms,cmhd->cshd", dS, Qc)   # [c, nk, H, D]
            dVg = np.einsum("chms,cmhd->cshd", P, dOc)
            sel = kb >= 0
            np.add.at(dK[b], kb[sel], dKg[sel])
            np.add.at(dV[b], kb[sel], dVg[sel])
    return dQ, dK, dV
