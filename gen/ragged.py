"""Seeded inputs for packed batches of images with different token counts.

The worked example of the English notes page "AFFMAE: Scalable Vision
Pre-Training for High-Resolution Microscopy Segmentation on Desktop
Hardware" ("A Complete Example") keeps *about* half of the 4096 patches
visible after Perlin masking; with a fixed noise level instead of a fixed
count every image keeps its own number of tokens, and a batch becomes a
packed ("varlen") set of images.  Recipes:

* "perlin_level": the three-octave gradient noise of :mod:`gen.synth`,
  every cell whose noise is above 0 is visible (row-major order), so the
  token count varies around half of the grid per image.
* "cells": ``lengths[b]`` distinct integer cells of a GxG grid drawn
  uniformly without replacement (token order as drawn).

One ``numpy.random.default_rng(seed)`` stream draws the geometry of every
image in order, then Q, K, V and dO as float32 standard normals [T, H, D]
(T = total tokens), converted to the workload dtype with RNE.  This module
holds no clustering or attention arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Union

import numpy as np

from .synth import _cells_xy, _gradient_noise, to_dtype


@dataclass(frozen=True)
class RaggedConfig:
    name: str
    seed: int
    B: int
    G: int
    H: int
    D: int
    dtype: str
    geometry: str                          # "perlin_level" | "cells"
    lengths: Optional[tuple] = None        # tokens per image ("cells" only)
    cs: int = 8
    k: int = 6

    @property
    def nk(self) -> int:
        return self.cs * self.k

    def with_batch(self, B: int) -> "RaggedConfig":
        lengths = None if self.lengths is None else self.lengths[:B]
        return replace(self, B=B, lengths=lengths)


RAGGED_CONFIGS = {
    # stage-1 geometry at a fixed noise level: 32 images of ~2048 tokens each
    "varlen": RaggedConfig("varlen", 4001, 32, 64, 4, 32, "bf16", "perlin_level"),
    # small sizes, empty and single-token images, one partial cluster each
    "varlen_tiny": RaggedConfig("varlen_tiny", 4002, 8, 32, 1, 32, "f32", "cells",
                                (1, 5, 8, 9, 63, 0, 300, 17)),
    # images above and below the in-LDS build limit of 2048 tokens, odd heads
    "varlen_mixed": RaggedConfig("varlen_mixed", 4003, 5, 128, 3, 32, "bf16", "cells",
                                 (2049, 3, 700, 4100, 16)),
}


def _level_cells(rng: np.random.Generator, G: int) -> np.ndarray:
    noise = np.zeros((G, G))
    for period, amp in ((16, 1.0), (8, 0.5), (4, 0.25)):
        noise += amp * _gradient_noise(rng, G, max(1, min(period, G)))
    return np.nonzero(noise.reshape(-1) > 0.0)[0]


def make_varlen_case(cfg: Union[str, RaggedConfig], B: int | None = None, tensors: bool = True):
    """Packed coordinates [T, 2] f32, per-image ``lengths`` and, when
    ``tensors``, Q, K, V, dO [T, H, D] as torch CPU tensors."""
    if isinstance(cfg, str):
        cfg = RAGGED_CONFIGS[cfg]
    if B is not None:
        cfg = cfg.with_batch(B)
    rng = np.random.default_rng(cfg.seed)
    pts, lengths = [], []
    for b in range(cfg.B):
        if cfg.geometry == "perlin_level":
            cells = _level_cells(rng, cfg.G)
        elif cfg.geometry == "cells":
            cells = rng.choice(cfg.G * cfg.G, size=cfg.lengths[b], replace=False)
        else:
            raise ValueError(cfg.geometry)
        pts.append(_cells_xy(cells, cfg.G))
        lengths.append(len(cells))
    coords = (np.concatenate(pts) if pts else np.zeros((0, 2))).astype(np.float32)
    case = {"cfg": cfg, "coords": coords, "lengths": lengths}
    if tensors:
        shape = (coords.shape[0], cfg.H, cfg.D)
        for name in ("q", "k", "v", "do"):
            case[name] = to_dtype(rng.standard_normal(shape, dtype=np.float32), cfg.dtype)
    return case
