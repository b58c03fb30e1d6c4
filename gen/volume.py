"""Seeded inputs for 3D (volumetric) tokens.

The notes page ("Limitations & Future Work") expects 3D voxels to carry
over without architectural change but gives no 3D workload.  The stand-ins
here mirror the 2D ones one dimension up: a 128^3 volume cut into 8^3
patches is a 16^3 patch grid of 4096 cells, of which a three-octave 3D
gradient-noise mask keeps the 2048 highest (the stage-1 token count), and a
fine-tune-like volume keeps every cell of a larger grid with sub-patch
jitter.  Recipes:

* "cells":  N distinct integer cells of a G^3 grid, uniformly without
  replacement (token order as drawn).
* "perlin3": three octaves of 3D gradient noise (lattice periods G/4, G/8,
  G/16 cells, amplitudes 1, 1/2, 1/4, uniformly random unit gradients, the
  quintic fade, trilinear blend), sampled at cell centres; the N highest
  cells are kept (ties to the lower flat index), flat order z-major, then
  y, then x.  With ``level`` set instead, every cell above that noise level
  is kept (a different count per volume).
* "jitter3": every cell of the G^3 grid at its centre plus U[-0.5, 0.5) per
  axis.

Coordinates are (x, y, z) in patch units; Q, K, V, dO are float32 standard
normals drawn after the geometry, converted with RNE.  No clustering or
attention arithmetic lives here.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Union

import numpy as np

from .synth import _fade, to_dtype


@dataclass(frozen=True)
class VolumeConfig:
    name: str
    seed: int
    B: int
    N: Optional[int]      # tokens per volume (None: by noise level)
    G: int
    H: int
    D: int
    dtype: str
    geometry: str         # "cells" | "perlin3" | "jitter3"
    level: Optional[float] = None
    cs: int = 8
    k: int = 6

    @property
    def nk(self) -> int:
        return self.cs * self.k

    @property
    def C(self) -> int:
        return -(-self.N // self.cs)

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def with_batch(self, B: int) -> "VolumeConfig":
        return replace(self, B=B)


VOLUME_CONFIGS = {
    "vol_tiny": VolumeConfig("vol_tiny", 5001, 1, 256, 8, 1, 32, "f32", "cells"),
    # 3D analogue of stage 1: 16^3 patch grid, 2048 visible tokens, 4 heads
    "volume": VolumeConfig("volume", 5002, 32, 2048, 16, 4, 32, "bf16", "perlin3"),
    # every cell of a 40^3 grid with jitter (64,000 tokens: the segment path)
    "volume_hr": VolumeConfig("volume_hr", 5003, 2, 64000, 40, 4, 32, "bf16", "jitter3"),
    # packed volumes, cells above noise level 0 (sizes differ per volume)
    "volume_varlen": VolumeConfig("volume_varlen", 5004, 6, None, 16, 2, 32, "bf16", "perlin3",
                                  level=0.0),
}


def _noise3(rng: np.random.Generator, G: int, period: int) -> np.ndarray:
    n = G // period + 2
    g = rng.standard_normal((n, n, n, 3))
    g /= np.linalg.norm(g, axis=-1, keepdims=True)
    c = (np.arange(G) + 0.5) / period
    z, y, x = np.meshgrid(c, c, c, indexing="ij")
    i0, j0, k0 = (np.floor(a).astype(np.int64) for a in (x, y, z))
    fx, fy, fz = x - i0, y - j0, z - k0

    def corner(di, dj, dk):
        gr = g[k0 + dk, j0 + dj, i0 + di]
        return gr[..., 0] * (fx - di) + gr[..., 1] * (fy - dj) + gr[..., 2] * (fz - dk)

    wx, wy, wz = _fade(fx), _fade(fy), _fade(fz)
    lerp = lambda a, b, t: a + t * (b - a)
    x00 = lerp(corner(0, 0, 0), corner(1, 0, 0), wx)
    x10 = lerp(corner(0, 1, 0), corner(1, 1, 0), wx)
    x01 = lerp(corner(0, 0, 1), corner(1, 0, 1), wx)
    x11 = lerp(corner(0, 1, 1), corner(1, 1, 1), wx)
    return lerp(lerp(x00, x10, wy), lerp(x01, x11, wy), wz)


def _perlin3(rng, G):
    noise = np.zeros((G, G, G))
    for div, amp in ((4, 1.0), (8, 0.5), (16, 0.25)):
        noise += amp * _noise3(rng, G, max(1, G // div))
    return noise.reshape(-1)


def _xyz(cells: np.ndarray, G: int) -> np.ndarray:
    return np.stack([cells % G, (cells // G) % G, cells // (G * G)], axis=1).astype(np.float64)


def make_volume_case(cfg: Union[str, VolumeConfig], B: int | None = None, tensors: bool = True):
    """Coordinates (equal sizes: [B, N, 3]; by level: packed [T, 3] with
    ``lengths``) and, when ``tensors``, Q, K, V, dO of matching shape."""
    if isinstance(cfg, str):
        cfg = VOLUME_CONFIGS[cfg]
    if B is not None:
        cfg = cfg.with_batch(B)
    rng = np.random.default_rng(cfg.seed)
    G = cfg.G
    pts = []
    for b in range(cfg.B):
        if cfg.geometry == "cells":
            xyz = _xyz(rng.choice(G ** 3, size=cfg.N, replace=False), G)
        elif cfg.geometry == "perlin3":
            noise = _perlin3(rng, G)
            if cfg.level is None:
                flat = np.arange(G ** 3)
                cells = np.sort(np.lexsort((flat, -noise))[:cfg.N])
            else:
                cells = np.nonzero(noise > cfg.level)[0]
            xyz = _xyz(cells, G)
        elif cfg.geometry == "jitter3":
            if cfg.N != G ** 3:
                raise ValueError("jitter3 covers the whole grid: N must be G^3")
            xyz = _xyz(np.arange(G ** 3), G) + rng.uniform(-0.5, 0.5, size=(cfg.N, 3))
        else:
            raise ValueError(cfg.geometry)
        pts.append(xyz.astype(np.float32))
    case = {"cfg": cfg}
    if cfg.N is None:
        case["lengths"] = [p.shape[0] for p in pts]
        case["coords"] = np.concatenate(pts) if pts else np.zeros((0, 3), np.float32)
        shape = (case["coords"].shape[0], cfg.H, cfg.D)
    else:
        case["coords"] = np.stack(pts) if pts else np.zeros((0, cfg.N, 3), np.float32)
        shape = (cfg.B, cfg.N, cfg.H, cfg.D)
    if tensors:
        for name in ("q", "k", "v", "do"):
            case[name] = to_dtype(rng.standard_normal(shape, dtype=np.float32), cfg.dtype)
    return case
