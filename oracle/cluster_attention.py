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
6. LSE is the natural log-sum-exp of the scaled logits.

Forward and backward are exact softmax attention, so the oracle writes the
plain definition (a count-masked dense form and an equivalent per-cluster
gathered form).  The neighbour build is a heuristic and is written as its
steps, in order.  All floating point is fp64; integer steps are exact.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "quantize",
    "morton_code",
    "balanced_clusters",
    "centroid_sums",
    "nearest_clusters",
    "nearest_clusters_fullsort",
    "key_lists",
    "build_neighbors",
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


def _sq_dist(S: np.ndarray, rows: np.ndarray) -> np.ndarray:
    dx = S[rows, 0][:, None] - S[None, :, 0]
    dy = S[rows, 1][:, None] - S[None, :, 1]
    return dx * dx + dy * dy  # exact int64: |d|^2 < 2**40


def nearest_clusters(S: np.ndarray, k: int, block: int = 512) -> np.ndarray:
    """Reading 4: slot 0 = self, then the k-1 other clusters with the smallest
    (squared centroid-sum distance, cluster index), ascending; -1 pads when
    the image has fewer than k clusters.  Returns [C, k] int64.

    Brute force over all clusters of the image; the (d2, index) pair is
    folded into one int64 key d2*C + index so the order is total."""
    C = S.shape[0]
    out = np.full((C, k), -1, dtype=np.int64)
    out[:, 0] = np.arange(C)
    take = min(k - 1, C - 1)
    if take <= 0:
        return out
    for r0 in range(0, C, block):
        rows = np.arange(r0, min(C, r0 + block))
        d2 = _sq_dist(S, rows)
        key = d2 * C + np.arange(C)[None, :]
        key[np.arange(rows.size), rows] = np.iinfo(np.int64).max  # exclude self
        part = np.argpartition(key, take - 1, axis=1)[:, :take]
        pk = np.take_along_axis(key, part, axis=1)
        order = np.argsort(pk, axis=1)
        out[rows, 1:1 + take] = np.take_along_axis(part, order, axis=1)
    return out


def nearest_clusters_fullsort(S: np.ndarray, k: int) -> np.ndarray:
    """Second formulation of reading 4 (used as a cross-check): a full
    lexicographic sort of all candidates of every cluster by (d2, index)."""
    C = S.shape[0]
    out = np.full((C, k), -1, dtype=np.int64)
    for c in range(C):
        dx = S[:, 0] - S[c, 0]
        dy = S[:, 1] - S[c, 1]
        d2 = dx * dx + dy * dy
        cand = np.array([b for b in range(C) if b != c], dtype=np.int64)
        order = cand[np.lexsort((cand, d2[cand]))]
        row = [c] + list(order[: k - 1])
        out[c, : len(row)] = row
    return out


def key_lists(perm: np.ndarray, nbr: np.ndarray, cs: int) -> tuple[np.ndarray, np.ndarray]:
    """q_idx[c, m] = perm[c*cs + m]; key_idx[c, s*cs + m] = perm[nbr[c,s]*cs + m]
    (or -1 where nbr is -1).  Returns int64 arrays [C, cs] and [C, k*cs]."""
    C, k = nbr.shape
    q_idx = perm.reshape(C, cs)
    key_idx = np.full((C, k * cs), -1, dtype=np.int64)
    for s in range(k):
        valid = nbr[:, s] >= 0
        key_idx[valid, s * cs:(s + 1) * cs] = q_idx[nbr[valid, s]]
    return q_idx, key_idx


def build_neighbors(coords: np.ndarray, grid_side: int, cs: int = 8, k: int = 6):
    """Whole neighbour build for a batch.

    coords [B, N, 2] float32  ->  perm [B, N], nbr [B, C, k],
    key_idx [B, C, k*cs], all int32 and image-local.  N must be a multiple
    of cs."""
    coords = np.asarray(coords)
    B, N, two = coords.shape
    assert two == 2 and N % cs == 0
    C = N // cs
    perm = np.empty((B, N), dtype=np.int32)
    nbr = np.empty((B, C, k), dtype=np.int32)
    key_idx = np.empty((B, C, k * cs), dtype=np.int32)
    for b in range(B):
        qx, qy = quantize(coords[b], grid_side)
        code = morton_code(qx, qy)
        p = balanced_clusters(code)
        S = centroid_sums(p, qx, qy, cs)
        nb = nearest_clusters(S, k)
        _, kl = key_lists(p, nb, cs)
        perm[b] = p
        nbr[b] = nb
        key_idx[b] = kl
    return perm, nbr, key_idx


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
            Qc = Q[b][qb]                      # [c, cs, H, D]
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
            O[b][qb] = Oc
            LSE[b][qb] = np.transpose(L, (0, 2, 1))
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
            Qc, dOc = Q[b][qb], dO[b][qb]          # [c, cs, H, D]
            Kg = _gather_rows(K[b], kb)            # [c, nk, H, D]
            Vg = _gather_rows(V[b], kb)
            S = scale * np.einsum("cmhd,cshd->chms", Qc, Kg)
            valid = (kb >= 0)[:, None, None, :]
            has = valid.any(axis=-1)
            m = np.where(has, np.where(valid, S, -np.inf).max(axis=-1), 0.0)
            E = np.where(valid, np.exp(S - m[..., None]), 0.0)
            Z = np.where(has, E.sum(axis=-1), 1.0)
            P = E / Z[..., None]                   # [c, H, cs, nk]
            Oc = np.einsum("chms,cshd->cmhd", P, Vg)
            delta = np.einsum("cmhd,cmhd->chm", dOc, Oc)
            dP = np.einsum("cmhd,cshd->chms", dOc, Vg)
            dS = P * (dP - delta[..., None])
            dQ[b][qb] = scale * np.einsum("chms,cshd->cmhd", dS, Kg)
            dKg = scale * np.einsum("chms,cmhd->cshd", dS, Qc)   # [c, nk, H, D]
            dVg = np.einsum("chms,cmhd->cshd", P, dOc)
            sel = kb >= 0
            np.add.at(dK[b], kb[sel], dKg[sel])
            np.add.at(dV[b], kb[sel], dVg[sel])
    return dQ, dK, dV
