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
    return TOL["stress"] if getattr(cfg, "qkv_scale", 1.0) != 1.0 else TOL[cfg.dtype]


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


def term_magnitudes(q, k, v, do, q_idx, key_idx, scale, cluster_block: int = 512):
    """Sums of the magnitudes of the terms that make up every output element,
    for floating-point error bars of the form u * sum|terms| (the standard
    bound for a rounded sum of products).  Returns fp64 arrays [B, N, H, D]:

      o:  sum_s P_ms |V_sd|
      dq: scale sum_s (|dS_ms| + P_ms E_m) |K_sd|
      dk: scale sum over the (m, s) holding key j of (|dS_ms| + P_ms E_m) |Q_md|
      dv: sum over the same (m, s) of P_ms |dO_md|

    with E_m = sum_d |dO_md| (|O_md| + o_md), which bounds (in units of u) the
    error of Delta_m = <dO_m, O_m> when O is the kernel's rounded output.
    P, dS are the exact (fp64) probabilities and their gradients, computed
    per cluster tile as in the gathered oracle.

    Also returns absolute floors, for operands rounded to fp16 below its
    normal range (|x| < 2^-14, absolute error up to 2^-25 whatever x is):
      o_floor:  sum_s |V_sd|            (unnormalised probabilities, <= 1,
                                          then divided by their sum >= 1)
      dq_floor: scale sum_s |K_sd|      (one dS per slot)
      dk_floor: scale sum over (m, s) holding j of |Q_md|
      dv_floor: sum over the same (m, s) of |dO_md|"""
    f = lambda x: x.detach().double().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    Q, K, V, dO = f(q), f(k), f(v), f(do)
    B, N, H, D = Q.shape
    names = ("o", "dq", "dk", "dv", "o_floor", "dq_floor", "dk_floor", "dv_floor")
    out = {n: np.zeros((B, N, H, D)) for n in names}

    def rows(X, idx):
        g = X[np.where(idx >= 0, idx, 0)]
        g[idx < 0] = 0.0
        return g

    for b in range(B):
        qi = np.asarray(q_idx[b]).astype(np.int64)
        ki = np.asarray(key_idx[b]).astype(np.int64)
        for c0 in range(0, qi.shape[0], cluster_block):
            qb, kb = qi[c0:c0 + cluster_block], ki[c0:c0 + cluster_block]
            Qc, dOc = rows(Q[b], qb), rows(dO[b], qb)
            Kg, Vg = rows(K[b], kb), rows(V[b], kb)
            S = scale * np.einsum("cmhd,cshd->chms", Qc, Kg)
            valid = (kb >= 0)[:, None, None, :]
            has = valid.any(axis=-1)
            m = np.where(has, np.where(valid, S, -np.inf).max(axis=-1), 0.0)
            E = np.where(valid, np.exp(S - m[..., None]), 0.0)
            P = E / np.where(has, E.sum(axis=-1), 1.0)[..., None]
            P = P * (qb >= 0)[:, None, :, None]
            Oc = np.einsum("chms,cshd->cmhd", P, Vg)
            magO = np.einsum("chms,cshd->cmhd", P, np.abs(Vg))
            delta = np.einsum("cmhd,cmhd->chm", dOc, Oc)
            dS = P * (np.einsum("cmhd,cshd->chms", dOc, Vg) - delta[..., None])
            Em = np.einsum("cmhd,cmhd->chm", np.abs(dOc), np.abs(Oc) + magO)
            W = np.abs(dS) + P * Em[..., None]
            live = qb >= 0
            out["o"][b][qb[live]] = magO[live]
            out["dq"][b][qb[live]] = scale * np.einsum("chms,cshd->cmhd", W, np.abs(Kg))[live]
            sel = kb >= 0
            np.add.at(out["dk"][b], kb[sel], (scale * np.einsum("chms,cmhd->cshd", W, np.abs(Qc)))[sel])
            np.add.at(out["dv"][b], kb[sel], np.einsum("chms,cmhd->cshd", P, np.abs(dOc))[sel])
            one = valid * (qb >= 0)[:, None, :, None] * np.ones_like(P)
            out["o_floor"][b][qb[live]] = np.einsum("chms,cshd->cmhd", one, np.abs(Vg))[live]
            out["dq_floor"][b][qb[live]] = scale * np.einsum("chms,cshd->cmhd", one,
                                                             np.abs(Kg))[live]
            np.add.at(out["dk_floor"][b], kb[sel],
                      (scale * np.einsum("chms,cmhd->cshd", one, np.abs(Qc)))[sel])
            np.add.at(out["dv_floor"][b], kb[sel], np.einsum("chms,cmhd->cshd", one, np.abs(dOc))[sel])
    return out
