"""Seeded generators for token geometry and attention inputs.

Every workload draws from one ``numpy.random.default_rng(seed)`` stream in
this order: the geometry of each image (in image order), then Q, K, V and dO
as float32 standard normals of shape [B, N, H, D].  The extra random choices
of the stress workload use a second stream seeded with (seed, 7) because they
act on neighbour lists that only exist after the build.  Conversion to bf16
or fp16 is round-to-nearest-even (torch ``.to``).

Geometry recipes (readings where the pages give only the idea):

* "cells":  N distinct integer cells of a GxG grid drawn uniformly without
  replacement, token order as drawn.
* "perlin": the structured mask of the English notes page "AFFMAE: Scalable
  Vision Pre-Training for High-Resolution Microscopy Segmentation on Desktop
  Hardware", "Key Designs" item 5 (Perlin masking) and "A Complete Example"
  (about half of 4096 patches visible).  Three octaves of 2D gradient noise
  with lattice periods 16, 8 and 4 cells and amplitudes 1, 1/2, 1/4, a
  uniformly random unit gradient per lattice point and the quintic fade
  6t^5-15t^4+10t^3, sampled at cell centres; the N highest cells are kept
  (ties to the lower flat index) and ordered row-major.
* "merged": stand-in for the adaptive merging of "Key Designs" item 1: a
  2048-cell Perlin set, N anchors drawn uniformly without replacement, every
  cell assigned to its nearest anchor (ties to the lower anchor), the token
  coordinate being the fp64 mean of its cells rounded to f32.
* "jitter": every cell of a GxG grid, row-major, at (col, row) plus
  U[-0.5, 0.5) per axis, rounded to f32.

Coordinates are (x = column, y = row) in patch units.
"""

from __future__ import annotations

import math
from typing import Union

import numpy as np

from .configs import CONFIGS, WorkloadConfig

_TORCH_DTYPES = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def to_dtype(x: np.ndarray, dtype: str):
    """float32 numpy array -> torch CPU tensor of ``dtype`` (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(getattr(torch, _TORCH_DTYPES[dtype]))


def _fade(t: np.ndarray) -> np.ndarray:
    return t * t * t * (t * (t * 6.0 - 15.0) + 10.0)


def _gradient_noise(rng: np.random.Generator, G: int, period: int) -> np.ndarray:
    """One octave of 2D gradient noise sampled at the centres of a GxG grid."""
    n = G // period + 2
    theta = rng.uniform(0.0, 2.0 * math.pi, size=(n, n))
    gx, gy = np.cos(theta), np.sin(theta)
    centres = (np.arange(G) + 0.5) / period
    u = centres[None, :].repeat(G, 0)      # x (column) in lattice units
    v = centres[:, None].repeat(G, 1)      # y (row)
    i0 = np.floor(u).astype(np.int64)
    j0 = np.floor(v).astype(np.int64)
    fu, fv = u - i0, v - j0

    def corner(di, dj):
        return gx[j0 + dj, i0 + di] * (fu - di) + gy[j0 + dj, i0 + di] * (fv - dj)

    n00, n10, n01, n11 = corner(0, 0), corner(1, 0), corner(0, 1), corner(1, 1)
    wu, wv = _fade(fu), _fade(fv)
    nx0 = n00 + wu * (n10 - n00)
    nx1 = n01 + wu * (n11 - n01)
    return nx0 + wv * (nx1 - nx0)


def perlin_visible_cells(rng: np.random.Generator, G: int, keep: int) -> np.ndarray:
    """Flat (row-major) ids of the ``keep`` cells with the highest noise."""
    noise = np.zeros((G, G))
    for period, amp in ((16, 1.0), (8, 0.5), (4, 0.25)):
        noise += amp * _gradient_noise(rng, G, max(1, min(period, G)))
    flat = np.arange(G * G)
    order = np.lexsort((flat, -noise.reshape(-1)))
    return np.sort(order[:keep])


def _cells_xy(cells: np.ndarray, G: int) -> np.ndarray:
    return np.stack([cells % G, cells // G], axis=1).astype(np.float64)


def _merged_coords(rng: np.random.Generator, G: int, n_tokens: int, n_visible: int = 2048) -> np.ndarray:
    cells = perlin_visible_cells(rng, G, n_visible)
    pts = _cells_xy(cells, G)
    anchors = rng.choice(n_visible, size=n_tokens, replace=False)
    apts = pts[anchors]
    d2 = ((pts[:, None, :] - apts[None, :, :]) ** 2).sum(-1)
    owner = np.argmin(d2, axis=1)          # first minimum = lower anchor index
    out = np.zeros((n_tokens, 2))
    for a in range(n_tokens):
        out[a] = pts[owner == a].mean(axis=0)
    return out


def make_coords(cfg: WorkloadConfig, rng: np.random.Generator) -> np.ndarray:
    """[B, N, 2] float32 coordinates for ``cfg`` (draws geometry per image)."""
    B, N, G = cfg.B, cfg.N, cfg.G
    out = np.empty((B, N, 2), dtype=np.float32)
    for b in range(B):
        if cfg.geometry == "cells":
            cells = rng.choice(G * G, size=N, replace=False)
            xy = _cells_xy(cells, G)
        elif cfg.geometry == "perlin":
            xy = _cells_xy(perlin_visible_cells(rng, G, N), G)
        elif cfg.geometry == "merged":
            xy = _merged_coords(rng, G, N, n_visible=min(2048, G * G))
        elif cfg.geometry == "jitter":
            if N != G * G:
                raise ValueError("jitter geometry covers the whole grid: N must be G*G")
            xy = _cells_xy(np.arange(G * G), G) + rng.uniform(-0.5, 0.5, size=(N, 2))
        else:
            raise ValueError(cfg.geometry)
        out[b] = xy.astype(np.float32)
    return out


def make_case(cfg: Union[str, WorkloadConfig], B: int | None = None, tensors: bool = True):
    """Coordinates and (optionally) Q, K, V, dO for one workload.

    Returns a dict with ``cfg``, ``coords`` (numpy f32 [B, N, 2]) and, when
    ``tensors``, ``q``, ``k``, ``v``, ``do`` as torch CPU tensors in the
    workload's dtype.  ``B`` overrides the batch (a smaller parity case of
    the same geometry)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if B is not None:
        cfg = cfg.with_batch(B)
    rng = np.random.default_rng(cfg.seed)
    case = {"cfg": cfg, "coords": make_coords(cfg, rng)}
    if tensors:
        shape = (cfg.B, cfg.N, cfg.H, cfg.D)
        z = [rng.standard_normal(shape, dtype=np.float32) for _ in range(4)]
        for name, arr in zip(("q", "k", "v"), z[:3]):
            case[name] = to_dtype(arr * np.float32(cfg.qkv_scale), cfg.dtype)
        case["do"] = to_dtype(z[3], cfg.dtype)
    return case


def stress_rng(cfg: WorkloadConfig) -> np.random.Generator:
    return np.random.default_rng((cfg.seed, 7))


def stress_duplicate_slots(key_idx: np.ndarray, cs: int, rng: np.random.Generator,
                           frac: float = 0.1, copies: int = 3) -> np.ndarray:
    """Copy 10% of the tokens of every image into the lists of 3 more clusters.

    For each image, round(frac*N) tokens are drawn; each goes into ``copies``
    clusters whose list does not hold it yet, overwriting one slot outside
    the cluster's own first ``cs`` slots that has not been overwritten
    before.  Entries inside a list stay distinct.  Returns a new int32 array.
    """
    out = np.array(key_idx, dtype=np.int32, copy=True)
    B, C, nk = out.shape
    N = C * cs
    for b in range(B):
        used = np.zeros((C, nk), dtype=bool)
        used[:, :cs] = True
        for t in rng.choice(N, size=int(round(frac * N)), replace=False):
            lacks = np.nonzero(~(out[b] == t).any(axis=1) & ~used.all(axis=1))[0]
            for c in rng.choice(lacks, size=min(copies, lacks.size), replace=False):
                free = np.nonzero(~used[c])[0]
                s = rng.choice(free)
                out[b, c, s] = t
                used[c, s] = True
    return out


def stress_copy_rows(k, v, rng: np.random.Generator, frac: float = 0.1):
    """The other reading of the stress workload: give round(frac*N) tokens per
    image the exact K and V rows of another token, creating equal logits.
    ``k``/``v`` are torch tensors [B, N, H, D]; returns modified clones."""
    k2, v2 = k.clone(), v.clone()
    B, N = k.shape[0], k.shape[1]
    n = int(round(frac * N))
    for b in range(B):
        dst = rng.choice(N, size=n, replace=False)
        src = rng.integers(0, N, size=n)
        src = np.where(src == dst, (src + 1) % N, src)
        k2[b, dst] = k[b, src]
        v2[b, dst] = v[b, src]
    return k2, v2
