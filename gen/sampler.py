"""Seeded inputs for the decoder's KNN-cache point sampler.

Shapes follow "A Complete Example" of the English notes page "AFFMAE:
Scalable Vision Pre-Training for High-Resolution Microscopy Segmentation on
Desktop Hardware": a 64x64 token grid, about 2048 visible tokens after
Perlin masking, stages of 2048 / 819 / 328 / 131 tokens with 128 / 256 / 512
/ 768 channels, and a decoder whose 2048 mask tokens are the queries, each
sampling every stage ("Key Designs" items 2 and 3).  Readings where the
pages are silent: K = 8 slots per table cell, p = 1 for every level,
query offsets uniform in [-1, 1) per axis (the offset net is not part of
the sampler), and the merged stages each built from the stage-1 visible set
by nearest-anchor means (not by repeated merging).

Draw order from ``numpy.random.default_rng(seed)``, per image: the Perlin
visible set, then the anchors of every merged level (in level order), then
the query offsets; after all images, per level: the features
[B, N, Cf] and the output gradients [B, M, Cf] as float32 standard normals,
converted to the workload dtype with round-to-nearest-even.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Tuple, Union

import numpy as np

from .synth import perlin_visible_cells, to_dtype


@dataclass(frozen=True)
class SamplerConfig:
    name: str
    seed: int
    B: int
    G: int
    M: int                                  # queries per image
    levels: Tuple[Tuple[int, int], ...]     # (tokens N, channels Cf) per level
    K: int
    p: float
    dtype: str                              # "f32" | "bf16" | "f16"
    geometry: str = "decoder"               # "decoder" | "uniform"

    def with_batch(self, B: int) -> "SamplerConfig":
        return replace(self, B=B)


SAMPLER_CONFIGS = {
    # small parity case: uniform tokens on a 16x16 grid, fp32, two levels
    "knn_tiny": SamplerConfig("knn_tiny", 2001, 2, 16, 96, ((40, 16), (7, 24)), 4, 1.5, "f32",
                              "uniform"),
    # the worked example's decoder sampling at pre-training batch 32
    "knn_decoder": SamplerConfig("knn_decoder", 2002, 32, 64, 2048,
                                 ((2048, 128), (819, 256), (328, 512), (131, 768)), 8, 1.0, "bf16"),
    # the same decoder on the 128 x 128 token grid of a 1024-pixel image
    # (half the cells visible, the other half queried)
    "knn_finetune": SamplerConfig("knn_finetune", 2003, 4, 128, 8192,
                                  ((8192, 128), (3277, 256), (1311, 512), (524, 768)), 8, 1.0,
                                  "bf16"),
    # and on a 256 x 256 grid (2048-pixel images)
    "knn_highres": SamplerConfig("knn_highres", 2004, 4, 256, 32768,
                                 ((32768, 128), (13107, 256), (5243, 512), (2097, 768)), 8, 1.0,
                                 "bf16"),
}


def _nearest_anchor_means(pts: np.ndarray, anchors: np.ndarray) -> np.ndarray:
    """Mean position of the points whose nearest anchor (smallest squared
    distance, then lower anchor index) is each anchor.  The points are
    integer cells, so squared distances and sums are exact; a k-d tree gives
    each point's nearest distance and every anchor within it, and the exact
    integer distances pick the owner among them."""
    from scipy.spatial import cKDTree

    apts = pts[anchors]
    tree = cKDTree(apts)
    dmin, _ = tree.query(pts, k=1)
    near = tree.query_ball_point(pts, dmin * (1 + 1e-9) + 1e-9)
    owner = np.empty(pts.shape[0], dtype=np.int64)
    for i, cand in enumerate(near):
        c = np.asarray(cand, dtype=np.int64)
        d2 = ((apts[c] - pts[i]) ** 2).sum(-1)
        owner[i] = c[d2 == d2.min()].min()
    cnt = np.bincount(owner, minlength=anchors.size).astype(np.float64)
    out = np.zeros((anchors.size, 2))
    for a in range(2):
        out[:, a] = np.bincount(owner, weights=pts[:, a], minlength=anchors.size) / cnt
    return out


def make_sampler_case(cfg: Union[str, SamplerConfig], B: int | None = None, tensors: bool = True):
    """Returns a dict with ``cfg``, ``coords`` (list per level of f32
    [B, N, 2]), ``queries`` (f32 [B, M, 2]) and, when ``tensors``,
    ``feats`` and ``dout`` (lists per level of torch CPU tensors)."""
    if isinstance(cfg, str):
        cfg = SAMPLER_CONFIGS[cfg]
    if B is not None:
        cfg = cfg.with_batch(B)
    rng = np.random.default_rng(cfg.seed)
    G, M = cfg.G, cfg.M
    coords = [np.empty((cfg.B, n, 2), dtype=np.float32) for n, _ in cfg.levels]
    queries = np.empty((cfg.B, M, 2), dtype=np.float32)
    for b in range(cfg.B):
        if cfg.geometry == "decoder":
            n1 = cfg.levels[0][0]
            vis = perlin_visible_cells(rng, G, n1)
            pts = np.stack([vis % G, vis // G], 1).astype(np.float64)
            coords[0][b] = pts.astype(np.float32)
            for li, (n, _) in enumerate(cfg.levels[1:], start=1):
                anchors = rng.choice(n1, size=n, replace=False)
                coords[li][b] = _nearest_anchor_means(pts, anchors).astype(np.float32)
            hidden = np.setdiff1d(np.arange(G * G), vis)
            r = np.stack([hidden % G, hidden // G], 1).astype(np.float64)
            if r.shape[0] < M:
                raise ValueError("fewer masked cells than queries")
            r = r[:M]
        else:   # uniform: tokens and queries anywhere in the grid
            for li, (n, _) in enumerate(cfg.levels):
                coords[li][b] = rng.uniform(-0.5, G - 0.5, size=(n, 2)).astype(np.float32)
            r = rng.uniform(-0.5, G - 0.5, size=(M, 2))
        queries[b] = (r + rng.uniform(-1.0, 1.0, size=(M, 2))).astype(np.float32)
    case = {"cfg": cfg, "coords": coords, "queries": queries}
    if tensors:
        case["feats"] = [to_dtype(rng.standard_normal((cfg.B, n, c), dtype=np.float32), cfg.dtype)
                         for n, c in cfg.levels]
        case["dout"] = [to_dtype(rng.standard_normal((cfg.B, M, c), dtype=np.float32), cfg.dtype)
                        for _, c in cfg.levels]
    return case
