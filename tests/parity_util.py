"""Helpers for the GPU parity tests (comparison against the fp64 oracle).

Tolerances (written here once, used by every parity test):
* fp32 inputs: max abs error <= 1e-5 on O, LSE and gradients.
* bf16 inputs: O <= 1e-2, dQ/dK/dV <= 2e-2, LSE <= 1e-3 (abs).
* fp16 large-logit stress: scale-relative, O <= 1e-2*max(1, max|O_ref|),
  gradients <= 2e-2*max(1, max|g_ref|), LSE <= 1e-2 abs; the absolute bars
  are below the fp16 output rounding of values that large.
* no NaN/Inf anywhere.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O

TOL = {
    "f32": dict(o=1e-5, lse=1e-5, g=1e-5, rel=False),
    "bf16": dict(o=1e-2, lse=1e-3, g=2e-2, rel=False),
    "f16": dict(o=1e-2, lse=1e-3, g=2e-2, rel=False),
    "stress": dict(o=1e-2, lse=1e-2, g=2e-2, rel=True),
}


def tol_for(cfg):
    return TOL["stress"] if cfg.qkv_scale != 1.0 else TOL[cfg.dtype]


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def assert_finite(name: str, t: torch.Tensor):
    bad = (~torch.isfinite(t.float())).sum().item()
    assert bad == 0, f"{name}: {bad} non-finite values"


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).max()) if got.size else 0.0


def check_close(name: str, got, ref: np.ndarray, tol: float, rel: bool):
    g = to_np(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    bar = tol * max(1.0, float(np.abs(ref).max())) if rel else tol
    err = max_err(g, ref)
    print(f"  {name}: max abs err {err:.3e} (bar {bar:.3e}, max|ref| {np.abs(ref).max():.3g})",
          flush=True)
    assert err <= bar, f"{name}: max abs error {err} > {bar}"


def referencing_clusters(key_idx_b: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """Clusters of one image whose key list holds any of ``tokens``."""
    return np.nonzero(np.isin(key_idx_b, tokens).any(axis=1))[0]


def sampled_oracle(q, k, v, do, q_idx, key_idx, scale, clusters, key_tokens, with_bwd=True):
    """Oracle outputs for one image restricted to some query clusters and to
    dK/dV rows of some key tokens (batch dim of 1).  Returns dict of arrays
    over the selected tokens."""
    qi = np.asarray(q_idx)
    ki = np.asarray(key_idx)
    out = {}
    sel_q = qi[clusters]
    o, lse = O.attn_fwd_gathered(q, k, v, sel_q[None], ki[clusters][None], scale)
    tok = sel_q.reshape(-1)
    tok = tok[tok >= 0]                      # -1: absent member of a partial cluster
    out["q_tokens"] = tok
    out["o"], out["lse"] = o[0, tok], lse[0, tok]
    if with_bwd:
        dq, _, _ = O.attn_bwd_gathered(q, k, v, do, sel_q[None], ki[clusters][None], scale)
        out["dq"] = dq[0, tok]
        refc = referencing_clusters(ki, key_tokens)
        _, dk, dv = O.attn_bwd_gathered(q, k, v, do, qi[refc][None], ki[refc][None], scale)
        out["k_tokens"] = key_tokens
        out["dk"], out["dv"] = dk[0, key_tokens], dv[0, key_tokens]
    return out
