"""GPU parity of the KNN-cache point sampler on fine-tune and high-resolution
grids (128 x 128 and 256 x 256 tokens; images above 4096 tokens take the
global-memory table build and the cursor-ranked backward lists), through
the C ABI, against the fp64 oracle.

* Tables bit-exact: every cell at 128 x 128, sampled cells at 256 x 256
  (the oracle ranks only the listed cells there).
* 128 x 128: outputs, feature gradients, query gradients and dp of whole
  images, element-wise, at the bars of the small-grid tests.
* 256 x 256 at the full four-image launch: outputs and query gradients of
  sampled queries (the oracle builds the table rows of their cells only),
  the feature-gradient sum rule (sum over tokens = sum over the queries of
  dout, the weights of a row summing to one), and a bitwise repeat of the
  backward (its lists are placed by atomics, then ranked)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from gen import make_sampler_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ca():
    import gathered_local_attention_amd as ca

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ca._lib.load()
    return ca


_CASES = {}


def _case(name, B=None):
    """Seeded cases, built once per module (the high-res one takes seconds)."""
    key = (name, B)
    if key not in _CASES:
        _CASES[key] = make_sampler_case(name, B=B)
    return _CASES[key]


def _bar(dtype, ref):
    rel = {torch.float32: 2e-6, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[dtype]
    return rel * np.abs(ref) + 2e-5 * max(1.0, float(np.abs(ref).max()))


def _check(name, got, ref, bar):
    err = np.abs(got - ref)
    worst = float((err - bar).max()) if err.size else -1.0
    print(f"  {name}: max abs err {float(err.max()) if err.size else 0:.3e} "
          f"(max|ref| {float(np.abs(ref).max()) if ref.size else 0:.3g})", flush=True)
    assert worst <= 0, f"{name}: error above bar by {worst:.3e}"


def _full_table(coords, G, K):
    ii, jj = np.meshgrid(np.arange(G), np.arange(G), indexing="ij")
    return O.knn_table_cells(coords, G, K, ii.reshape(-1), jj.reshape(-1)).reshape(G, G, K)


def _dq_bar(dq_ref):
    return 2e-4 * max(1.0, float(np.abs(dq_ref).max())) + 1e-3 * np.abs(dq_ref)


@pytest.mark.parametrize("li,B", [(0, 2), (1, 1), (2, 1), (3, 1)])
def test_finetune_levels_whole_images(ca, li, B):
    case = _case("knn_finetune", B)
    cfg = case["cfg"]
    N, C = cfg.levels[li]
    print(f"case knn_finetune B={B} level {li} (N={N}, C={C})", flush=True)
    coords, q = case["coords"][li], case["queries"]
    feats, dout = case["feats"][li], case["dout"][li]
    dc = torch.from_numpy(coords).to(DEV)
    dq_in = torch.from_numpy(q).to(DEV)
    table = ca.knn_table(dc, cfg.G, cfg.K)
    df = feats.to(DEV)
    out = ca.knn_sample_fwd(df, dc, dq_in, table, cfg.p)
    dF, dqg, dp = ca.knn_sample_bwd(df, dc, dq_in, table, cfg.p, dout.to(DEV))
    torch.cuda.synchronize()
    F64, dO64 = feats.double().numpy(), dout.double().numpy()
    dp_ref = 0.0
    for b in range(B):
        t_ref = _full_table(coords[b], cfg.G, cfg.K)
        diff = np.argwhere(table[b].cpu().numpy() != t_ref)
        assert diff.size == 0, f"image {b}: {len(diff)} table mismatches, first {diff[:3].tolist()}"
        o_ref = O.knn_sample_fwd(coords[b], F64[b], q[b], t_ref, cfg.p)
        _check(f"b{b} out", out[b].double().cpu().numpy(), o_ref, _bar(feats.dtype, o_ref))
        dF_ref, dq_ref, dp_b = O.knn_sample_bwd(coords[b], F64[b], q[b], t_ref, cfg.p, dO64[b])
        dp_ref += dp_b
        _check(f"b{b} dF", dF[b].double().cpu().numpy(), dF_ref, _bar(feats.dtype, dF_ref))
        _check(f"b{b} dq", dqg[b].double().cpu().numpy(), dq_ref, _dq_bar(dq_ref))
    _check("dp", np.array([float(dp.item())]), np.array([dp_ref]),
           np.array([1e-4 * max(1.0, abs(dp_ref)) + 1e-4 * np.sqrt(B * cfg.M * cfg.K)]))


def _sparse_table(coords, G, K, rows, cols):
    """[G, G, K] with the oracle's rows at the listed cells, -1 elsewhere."""
    t = np.full((G, G, K), -1, dtype=np.int64)
    cells = np.unique(rows * G + cols)
    r, c = cells // G, cells % G
    t[r, c] = O.knn_table_cells(coords, G, K, r, c)
    return t


@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_highres_full_launch_sampled(ca, li):
    case = _case("knn_highres")
    cfg = case["cfg"]
    N, C = cfg.levels[li]
    G, K = cfg.G, cfg.K
    print(f"case knn_highres B={cfg.B} level {li} (N={N}, C={C})", flush=True)
    coords, q = case["coords"][li], case["queries"]
    feats, dout = case["feats"][li], case["dout"][li]
    dc = torch.from_numpy(coords).to(DEV)
    dq_in = torch.from_numpy(q).to(DEV)
    table = ca.knn_table(dc, G, K)
    df, ddo = feats.to(DEV), dout.to(DEV)
    out = ca.knn_sample_fwd(df, dc, dq_in, table, cfg.p)
    dF, dqg, dp = ca.knn_sample_bwd(df, dc, dq_in, table, cfg.p, ddo)
    dF2, dqg2, dp2 = ca.knn_sample_bwd(df, dc, dq_in, table, cfg.p, ddo)
    torch.cuda.synchronize()
    assert torch.equal(dF, dF2) and torch.equal(dqg, dqg2) and torch.equal(dp, dp2), "not bitwise repeatable"
    rng = np.random.default_rng(7000 + li)
    F64, dO64 = feats.double().numpy(), dout.double().numpy()
    for b in range(cfg.B):
        # table: the four corners, the border rows and columns, random cells
        rr = np.concatenate([[0, 0, G - 1, G - 1], np.zeros(G, int), np.full(G, G - 1),
                             np.arange(G), rng.integers(0, G, 1500)])
        cc = np.concatenate([[0, G - 1, 0, G - 1], np.arange(G), np.arange(G),
                             np.full(G, G // 2), rng.integers(0, G, 1500)])
        t_ref = O.knn_table_cells(coords[b], G, K, rr, cc)
        t_gpu = table[b].cpu().numpy()[rr, cc]
        bad = np.argwhere(t_gpu != t_ref)
        assert bad.size == 0, f"image {b}: {len(bad)} table mismatches at cells " \
                              f"{[(int(rr[i]), int(cc[i])) for i, _ in bad[:3]]}"
        # sampled queries: out and dq from the oracle's own rows of their cells
        sel = np.sort(rng.choice(cfg.M, size=1024, replace=False))
        qi, qj = O.query_cells(q[b, sel], G)
        t_sp = _sparse_table(coords[b], G, K, qi, qj)
        o_ref = O.knn_sample_fwd(coords[b], F64[b], q[b, sel], t_sp, cfg.p)
        _check(f"b{b} out (1024 queries)", out[b, sel].double().cpu().numpy(), o_ref,
               _bar(feats.dtype, o_ref))
        _, dq_ref, _ = O.knn_sample_bwd(coords[b], F64[b], q[b, sel], t_sp, cfg.p, dO64[b, sel])
        _check(f"b{b} dq (1024 queries)", dqg[b, sel].double().cpu().numpy(), dq_ref, _dq_bar(dq_ref))
        # sum rule: every query has K >= 1 valid slots (N >= K), weights sum to 1
        got = dF[b].double().sum(0).cpu().numpy()
        ref = dO64[b].sum(0)
        bar = 2.0 ** -8 * dF[b].double().abs().sum(0).cpu().numpy() + 1e-3
        _check(f"b{b} sum_t dF", got, ref, bar)


@pytest.mark.parametrize("G,K,N", [(100, 16, 5000), (256, 8, 20000), (2048, 1, 4097), (3, 5, 6000)])
def test_large_table_edge_shapes(ca, G, K, N):
    """Images above 4096 tokens: G not a power of two with K = 16, the
    largest grid with one slot, a three-cell grid holding many tokens per
    cell; coordinates outside the grid and repeated ones (distance ties)."""
    rng = np.random.default_rng(G * 7 + K + N)
    pts = rng.uniform(-3.0, G + 2.0, size=(2, N, 2)).astype(np.float32)
    pts[:, N // 2:] = pts[:, : N - N // 2]
    print(f"case large table G={G} K={K} N={N}", flush=True)
    table = ca.knn_table(torch.from_numpy(pts).to(DEV), G, K).cpu().numpy()
    for b in range(2):
        if G * G <= 16384:
            ref = _full_table(pts[b], G, K)
            assert np.array_equal(table[b], ref), f"image {b}"
        else:
            rr = rng.integers(0, G, 2000)
            cc = rng.integers(0, G, 2000)
            rr[:4], cc[:4] = [0, 0, G - 1, G - 1], [0, G - 1, 0, G - 1]
            ref = O.knn_table_cells(pts[b], G, K, rr, cc)
            assert np.array_equal(table[b][rr, cc], ref), f"image {b}"


def test_large_backward_uncovered_tokens_get_zero(ca):
    """Queries that all fall in one corner: the tokens no query reaches get
    a zero feature gradient, the rest match the oracle."""
    G, K, C, N, M = 96, 4, 32, 6000, 300
    rng = np.random.default_rng(11)
    pts = rng.uniform(-0.5, G - 0.5, size=(1, N, 2)).astype(np.float32)
    q = rng.uniform(0, 6, size=(1, M, 2)).astype(np.float32)
    F = rng.standard_normal((1, N, C)).astype(np.float32)
    dO = rng.standard_normal((1, M, C)).astype(np.float32)
    dc = torch.from_numpy(pts).to(DEV)
    table = ca.knn_table(dc, G, K)
    dF, dq, dp = ca.knn_sample_bwd(torch.from_numpy(F).to(DEV), dc, torch.from_numpy(q).to(DEV),
                                   table, 0.7, torch.from_numpy(dO).to(DEV))
    qi, qj = O.query_cells(q[0], G)
    t_sp = _sparse_table(pts[0], G, K, qi, qj)
    dF_ref, dq_ref, dp_ref = O.knn_sample_bwd(pts[0], F[0].astype(np.float64), q[0], t_sp, 0.7,
                                              dO[0].astype(np.float64))
    _check("dF", dF[0].double().cpu().numpy(), dF_ref, _bar(torch.float32, dF_ref))
    _check("dq", dq[0].double().cpu().numpy(), dq_ref, _dq_bar(dq_ref))
    _check("dp", np.array([float(dp.item())]), np.array([dp_ref]),
           np.array([1e-4 * max(1.0, abs(dp_ref)) + 1e-4 * np.sqrt(M * K)]))
    assert int((dF_ref == 0).all(axis=1).sum()) > N - 200


def test_large_backward_token_with_thousands_of_entries(ca):
    """Every query in one corner and K = 16: the corner tokens hold thousands
    of entries each (their lists go through the stable long-segment sort,
    the others through the ranking); everything against the oracle."""
    G, K, C, N, M = 80, 16, 32, 5000, 4000
    rng = np.random.default_rng(21)
    pts = rng.uniform(-0.5, G - 0.5, size=(1, N, 2)).astype(np.float32)
    q = rng.uniform(0, 2.5, size=(1, M, 2)).astype(np.float32)
    F = rng.standard_normal((1, N, C)).astype(np.float32)
    dO = rng.standard_normal((1, M, C)).astype(np.float32)
    dc = torch.from_numpy(pts).to(DEV)
    table = ca.knn_table(dc, G, K)
    dF, dq, dp = ca.knn_sample_bwd(torch.from_numpy(F).to(DEV), dc, torch.from_numpy(q).to(DEV),
                                   table, 1.1, torch.from_numpy(dO).to(DEV))
    dF2, _, _ = ca.knn_sample_bwd(torch.from_numpy(F).to(DEV), dc, torch.from_numpy(q).to(DEV),
                                  table, 1.1, torch.from_numpy(dO).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(dF, dF2), "not bitwise repeatable"
    qi, qj = O.query_cells(q[0], G)
    t_sp = _sparse_table(pts[0], G, K, qi, qj)
    counts = np.bincount(t_sp[qi, qj].reshape(-1), minlength=N)
    print(f"  most entries of one token: {counts.max()}", flush=True)
    assert counts.max() > 1024
    dF_ref, dq_ref, dp_ref = O.knn_sample_bwd(pts[0], F[0].astype(np.float64), q[0], t_sp, 1.1,
                                              dO[0].astype(np.float64))
    _check("dF", dF[0].double().cpu().numpy(), dF_ref, _bar(torch.float32, dF_ref))
    _check("dq", dq[0].double().cpu().numpy(), dq_ref, _dq_bar(dq_ref))
    _check("dp", np.array([float(dp.item())]), np.array([dp_ref]),
           np.array([1e-4 * max(1.0, abs(dp_ref)) + 1e-4 * np.sqrt(M * K)]))
