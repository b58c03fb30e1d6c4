"""Seeded inputs for adaptive off-grid token merging.

Shapes follow "A Complete Example" of the English notes page "AFFMAE:
Scalable Vision Pre-Training for High-Resolution Microscopy Segmentation on
Desktop Hardware": at retention 0.4 the stages keep 2048 -> 819 -> 328 ->
131 tokens with 128 / 256 / 512 channels before each merge, at pre-training
batch 32 ("Key Designs" item 1 for the merge itself).  Readings where the
pages are silent: the importance scores (the output of the scoring MLP) are
standard normals; the first level's tokens are the Perlin-visible cells of
the 64x64 grid (every cell of the grid for the fine-tune workloads, which
see whole images), the later levels' tokens the nearest-anchor means of
that set (as the stage-3 workload of the attention benchmarks).

Draw order from ``numpy.random.default_rng(seed)``: per image the Perlin
set and, for the later levels, their anchors; then per level the scores
[B, N], the features [B, N, C], the output gradients [B, k, C] and
[B, k, 2], all float32 standard normals (features and dF' rounded to the
workload dtype, round-to-nearest-even).
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Tuple, Union

import numpy as np

from .sampler import _nearest_anchor_means
from .synth import perlin_visible_cells, to_dtype


@dataclass(frozen=True)
class MergeConfig:
    name: str
    seed: int
    B: int
    G: int
    levels: Tuple[Tuple[int, int, int], ...]   # (tokens N, anchors k, channels C)
    dtype: str

    def with_batch(self, B: int) -> "MergeConfig":
        return replace(self, B=B)


MERGE_CONFIGS = {
    "merge_tiny": MergeConfig("merge_tiny", 3001, 2, 16, ((60, 23, 16), (23, 9, 24)), "f32"),
    "merge_stages": MergeConfig("merge_stages", 3002, 32, 64,
                                ((2048, 819, 128), (819, 328, 256), (328, 131, 512)), "bf16"),
    # fine-tuning sees every token: the full 128 x 128 grid of a 1024-pixel
    # image, and the 256 x 256 grid of a 2048-pixel one, at retention 0.4
    "merge_finetune": MergeConfig("merge_finetune", 3003, 4, 128,
                                  ((16384, 6554, 128), (6554, 2622, 256), (2622, 1049, 512)),
                                  "bf16"),
    "merge_highres": MergeConfig("merge_highres", 3004, 4, 256,
                                 ((65536, 26214, 128), (26214, 10486, 256), (10486, 4194, 512)),
                                 "bf16"),
}


def make_merge_case(cfg: Union[str, MergeConfig], B: int | None = None, tensors: bool = True):
    """Returns a dict with ``cfg``, ``coords`` (list per level of f32
    [B, N, 2]), ``scores`` (list of f32 [B, N]) and, when ``tensors``,
    ``feats``, ``dfeat`` (lists of torch CPU tensors) and ``dcoord`` (list
    of f32 [B, k, 2])."""
    if isinstance(cfg, str):
        cfg = MERGE_CONFIGS[cfg]
    if B is not None:
        cfg = cfg.with_batch(B)
    rng = np.random.default_rng(cfg.seed)
    G = cfg.G
    coords = [np.empty((cfg.B, n, 2), dtype=np.float32) for n, _, _ in cfg.levels]
    for b in range(cfg.B):
        n1 = cfg.levels[0][0]
        if n1 == G * G:          # every cell of the grid, row-major
            cells = np.arange(G * G)
            pts = np.stack([cells % G, cells // G], 1).astype(np.float64)
        elif n1 <= G * G // 2:
            vis = perlin_visible_cells(rng, G, n1)
            pts = np.stack([vis % G, vis // G], 1).astype(np.float64)
        else:
            pts = rng.uniform(-0.5, G - 0.5, size=(n1, 2))
        coords[0][b] = pts.astype(np.float32)
        for li, (n, _, _) in enumerate(cfg.levels[1:], start=1):
            anchors = rng.choice(n1, size=n, replace=False)
            coords[li][b] = _nearest_anchor_means(pts, anchors).astype(np.float32)
    scores = [rng.standard_normal((cfg.B, n), dtype=np.float32) for n, _, _ in cfg.levels]
    case = {"cfg": cfg, "coords": coords, "scores": scores}
    if tensors:
        case["feats"] = [to_dtype(rng.standard_normal((cfg.B, n, c), dtype=np.float32), cfg.dtype)
                         for n, _, c in cfg.levels]
        case["dfeat"] = [to_dtype(rng.standard_normal((cfg.B, k, c), dtype=np.float32), cfg.dtype)
                         for _, k, c in cfg.levels]
        case["dcoord"] = [rng.standard_normal((cfg.B, k, 2), dtype=np.float32) for _, k, _ in cfg.levels]
    return case
