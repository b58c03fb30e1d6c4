"""Pins of the oracle's attention forward/backward against textbook dense
attention (torch CPU fp64), autograd, finite differences, closed forms and
invariants (no GPU)."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from gen import make_case, stress_duplicate_slots
from gen.synth import stress_rng


def _random_lists(rng, N, cs, nk, repeats=True, holes=True):
    """Random cluster partition and random key lists, with optional repeated
    slots and -1 holes (every list keeps at least one valid slot)."""
    perm = rng.permutation(N)
    C = N // cs
    q_idx = perm.reshape(C, cs)
    key_idx = rng.integers(0, N, size=(C, nk))
    if repeats:
        key_idx[:, 1] = key_idx[:, 0]
        key_idx[::3, 2] = key_idx[::3, 0]
    if holes:
        key_idx[:, -1] = -1
        key_idx[1::2, -2] = -1
    return q_idx[None], key_idx[None]


def _textbook(q, k, v, q_idx, key_idx, scale):
    """Dense attention through torch's SDPA with an additive float mask
    log(count) (count 0 -> -inf): the textbook form of slot multiplicity."""
    B, N, H, D = q.shape
    M = np.stack([O.count_matrix(q_idx[b], key_idx[b], N) for b in range(B)])
    with np.errstate(divide="ignore"):
        bias = torch.from_numpy(np.log(M))                 # [B, N, N]
    qt = torch.as_tensor(q, dtype=torch.float64).permute(0, 2, 1, 3)
    kt = torch.as_tensor(k, dtype=torch.float64).permute(0, 2, 1, 3)
    vt = torch.as_tensor(v, dtype=torch.float64).permute(0, 2, 1, 3)
    return qt, kt, vt, bias[:, None]


def _sdpa(qt, kt, vt, mask, scale):
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)


def test_full_neighbourhood_equals_dense_textbook():
    """k = C: every cluster lists every token, so the method is full
    softmax attention over all N tokens."""
    rng = np.random.default_rng(1)
    B, N, H, D, cs = 2, 64, 2, 16, 8
    q, k, v = (rng.standard_normal((B, N, H, D)) for _ in range(3))
    q_idx = np.stack([rng.permutation(N).reshape(-1, cs) for _ in range(B)])
    key_idx = np.stack([np.tile(rng.permutation(N), (N // cs, 1)) for _ in range(B)])
    scale = 1 / math.sqrt(D)
    qt, kt, vt = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = _sdpa(qt, kt, vt, None, scale).permute(0, 2, 1, 3).numpy()
    ref_lse = torch.logsumexp(scale * qt @ kt.transpose(-1, -2), dim=-1).permute(0, 2, 1).numpy()
    for fn in (O.attn_fwd_dense, O.attn_fwd_gathered):
        o, lse = fn(q, k, v, q_idx, key_idx, scale)
        assert np.abs(o - ref).max() <= 1e-12
        assert np.abs(lse - ref_lse).max() <= 1e-12


def test_multiplicity_and_holes_equal_log_count_bias():
    rng = np.random.default_rng(2)
    N, H, D, cs, nk = 64, 2, 8, 8, 24
    q_idx, key_idx = _random_lists(rng, N, cs, nk)
    q, k, v = (rng.standard_normal((1, N, H, D)) for _ in range(3))
    scale = 0.3
    qt, kt, vt, mask = _textbook(q, k, v, q_idx, key_idx, scale)
    ref = _sdpa(qt, kt, vt, mask, scale).permute(0, 2, 1, 3).numpy()
    ref_lse = torch.logsumexp(scale * qt @ kt.transpose(-1, -2) + mask, dim=-1).permute(0, 2, 1).numpy()
    for fn in (O.attn_fwd_dense, O.attn_fwd_gathered):
        o, lse = fn(q, k, v, q_idx, key_idx, scale)
        assert np.abs(o - ref).max() <= 1e-12
        assert np.abs(lse - ref_lse).max() <= 1e-12


def test_backward_equals_autograd_of_textbook():
    rng = np.random.default_rng(3)
    N, H, D, cs, nk = 64, 2, 8, 8, 24
    q_idx, key_idx = _random_lists(rng, N, cs, nk)
    q, k, v, do = (rng.standard_normal((1, N, H, D)) for _ in range(4))
    scale = 0.35
    qt, kt, vt, mask = _textbook(q, k, v, q_idx, key_idx, scale)
    for t in (qt, kt, vt):
        t.requires_grad_(True)
    out = _sdpa(qt, kt, vt, mask, scale)
    out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    refs = [t.grad.permute(0, 2, 1, 3).numpy() for t in (qt, kt, vt)]
    for fn in (O.attn_bwd_dense, O.attn_bwd_gathered):
        grads = fn(q, k, v, do, q_idx, key_idx, scale)
        for g, r in zip(grads, refs):
            assert np.abs(g - r).max() <= 1e-12


def test_backward_finite_differences():
    rng = np.random.default_rng(4)
    N, H, D, cs, nk = 32, 2, 8, 8, 16
    q_idx, key_idx = _random_lists(rng, N, cs, nk)
    q, k, v, do = (rng.standard_normal((1, N, H, D)) for _ in range(4))
    scale = 1 / math.sqrt(D)
    grads = O.attn_bwd_gathered(q, k, v, do, q_idx, key_idx, scale)

    def loss(qq, kk, vv):
        o, _ = O.attn_fwd_dense(qq, kk, vv, q_idx, key_idx, scale)
        return float((o * do).sum())

    h = 1e-6
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        for _ in range(40):
            idx = tuple(rng.integers(0, s) for s in q.shape)
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            an = grads[which][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, idx, fd, an)


def test_zero_queries_give_uniform_average():
    rng = np.random.default_rng(5)
    N, H, D, cs, nk = 64, 1, 8, 8, 24
    q_idx, key_idx = _random_lists(rng, N, cs, nk)
    q = np.zeros((1, N, H, D))
    k, v = (rng.standard_normal((1, N, H, D)) for _ in range(2))
    o, lse = O.attn_fwd_gathered(q, k, v, q_idx, key_idx, 0.5)
    for c in range(N // cs):
        valid = key_idx[0, c][key_idx[0, c] >= 0]
        mean_v = v[0, valid].mean(axis=0)
        for i in q_idx[0, c]:
            assert np.abs(o[0, i] - mean_v).max() <= 1e-12
            assert abs(lse[0, i, 0] - math.log(valid.size)) <= 1e-12


def test_key_shift_moves_only_lse():
    rng = np.random.default_rng(6)
    N, H, D, cs, nk = 64, 2, 8, 8, 24
    q_idx, key_idx = _random_lists(rng, N, cs, nk)
    q, k, v = (rng.standard_normal((1, N, H, D)) for _ in range(3))
    w = rng.standard_normal((H, D)) * 400.0         # logit shifts of ~1e3
    scale = 0.4
    o1, l1 = O.attn_fwd_gathered(q, k, v, q_idx, key_idx, scale)
    o2, l2 = O.attn_fwd_gathered(q, k + w[None, None], v, q_idx, key_idx, scale)
    shift = scale * np.einsum("bnhd,hd->bnh", q, w)
    assert np.abs(o1 - o2).max() <= 1e-10
    assert np.abs((l2 - l1 - shift) / np.maximum(1.0, np.abs(l2))).max() <= 1e-12


def test_gradient_sum_rules():
    rng = np.random.default_rng(7)
    N, H, D, cs, nk = 64, 2, 8, 8, 24
    q_idx, key_idx = _random_lists(rng, N, cs, nk)
    q, k, v, do = (rng.standard_normal((1, N, H, D)) for _ in range(4))
    dq, dk, dv = O.attn_bwd_gathered(q, k, v, do, q_idx, key_idx, 0.3)
    assert np.abs(dk.sum(axis=1)).max() <= 1e-10
    assert np.abs(dv.sum(axis=1) - do.sum(axis=1)).max() <= 1e-10


def test_permutation_within_clusters_and_lists():
    rng = np.random.default_rng(8)
    N, H, D, cs, nk = 64, 2, 8, 8, 24
    q_idx, key_idx = _random_lists(rng, N, cs, nk)
    q, k, v, do = (rng.standard_normal((1, N, H, D)) for _ in range(4))
    o1, l1 = O.attn_fwd_gathered(q, k, v, q_idx, key_idx, 0.3)
    g1 = O.attn_bwd_gathered(q, k, v, do, q_idx, key_idx, 0.3)
    q2 = np.stack([rng.permutation(r) for r in q_idx[0]])[None]
    k2 = np.stack([rng.permutation(r) for r in key_idx[0]])[None]
    o2, l2 = O.attn_fwd_gathered(q, k, v, q2, k2, 0.3)
    g2 = O.attn_bwd_gathered(q, k, v, do, q2, k2, 0.3)
    assert np.abs(o1 - o2).max() <= 1e-12 and np.abs(l1 - l2).max() <= 1e-12
    for a, b in zip(g1, g2):
        assert np.abs(a - b).max() <= 1e-12


def test_token_relabelling_permutes_outputs():
    case = make_case("stage3", B=1)
    cfg = case["cfg"]
    scale = cfg.D ** -0.5
    pi = np.random.default_rng(9).permutation(cfg.N)
    inv = np.argsort(pi)
    p1, _, k1 = O.build_neighbors(case["coords"], cfg.G)
    p2, _, k2 = O.build_neighbors(case["coords"][:, pi], cfg.G)
    o1, l1 = O.attn_fwd_gathered(case["q"], case["k"], case["v"], p1.reshape(1, -1, 8), k1, scale)
    qs, ks, vs = (case[n][:, pi] for n in ("q", "k", "v"))
    o2, l2 = O.attn_fwd_gathered(qs, ks, vs, p2.reshape(1, -1, 8), k2, scale)
    assert np.abs(o2[:, inv] - o1).max() <= 1e-12
    assert np.abs(l2[:, inv] - l1).max() <= 1e-12


@pytest.mark.parametrize("name,B", [("tiny", None), ("stage1", 1), ("stage3", 1), ("stress", 1)])
def test_gathered_equals_dense(name, B):
    case = make_case(name, B=B)
    cfg = case["cfg"]
    perm, _, key_idx = O.build_neighbors(case["coords"], cfg.G)
    if cfg.dup_frac:
        key_idx = stress_duplicate_slots(key_idx, cfg.cs, stress_rng(cfg), cfg.dup_frac)
    q_idx = perm.reshape(cfg.B, cfg.C, cfg.cs)
    scale = cfg.D ** -0.5
    H = min(cfg.H, 2)
    args = [case[n][:, :, :H] for n in ("q", "k", "v")]
    od, ld = O.attn_fwd_dense(*args, q_idx, key_idx, scale)
    og, lg = O.attn_fwd_gathered(*args, q_idx, key_idx, scale)
    tol = 1e-12 * max(1.0, float(np.abs(ld).max()))
    assert np.abs(od - og).max() <= 1e-12 * max(1.0, float(np.abs(od).max()))
    assert np.abs(ld - lg).max() <= tol
    if cfg.passes == "fwd+bwd":
        do = case["do"][:, :, :H]
        gd = O.attn_bwd_dense(*args, do, q_idx, key_idx, scale)
        gg = O.attn_bwd_gathered(*args, do, q_idx, key_idx, scale)
        for a, b in zip(gd, gg):
            assert np.abs(a - b).max() <= 1e-11 * max(1.0, float(np.abs(a).max()))


def test_stress_duplicates_follow_their_recipe():
    case = make_case("stress", B=2, tensors=False)
    cfg = case["cfg"]
    _, _, key_idx = O.build_neighbors(case["coords"], cfg.G)
    dup = stress_duplicate_slots(key_idx, cfg.cs, stress_rng(cfg), cfg.dup_frac)
    changed = dup != key_idx
    assert not changed[:, :, :cfg.cs].any()
    assert changed.sum() == cfg.B * 3 * round(0.1 * cfg.N)
    for b in range(cfg.B):
        for c in range(cfg.C):
            assert len(set(dup[b, c])) == cfg.nk


def test_generators_are_deterministic():
    a = make_case("stage3", B=2)
    b = make_case("stage3", B=2)
    assert np.array_equal(a["coords"], b["coords"])
    for n in ("q", "k", "v", "do"):
        assert torch.equal(a[n], b[n])
    s = make_case("stress", B=1)
    assert s["q"].dtype == torch.float16 and s["q"].abs().max() > 20
    p = make_case("stage1", B=2, tensors=False)["coords"]
    for img in p:
        cells = set(map(tuple, img.astype(int)))
        assert len(cells) == 2048 and img.min() >= 0 and img.max() <= 63
