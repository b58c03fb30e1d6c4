"""GPU parity of the KNN-cache point sampler against the fp64 oracle, through
the C ABI.  Tables must match bit-exactly; sampled features, feature
gradients, query gradients and dp within the bars below (derived from the
arithmetic: fp32 accumulation everywhere, one RNE rounding of bf16 outputs,
|relative error| <= 2^-9, plus fp32 error of the weights)."""

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


def _bar(dtype, ref):
    """Element-wise bar: fp32 arithmetic, plus the output rounding of bf16/fp16."""
    rel = {torch.float32: 2e-6, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[dtype]
    return rel * np.abs(ref) + 2e-5 * max(1.0, float(np.abs(ref).max()))


def _check(name, got, ref, bar):
    err = np.abs(got - ref)
    worst = float((err - bar).max()) if err.size else -1.0
    print(f"  {name}: max abs err {float(err.max()) if err.size else 0:.3e} "
          f"(max|ref| {float(np.abs(ref).max()) if ref.size else 0:.3g})", flush=True)
    assert worst <= 0, f"{name}: error above bar by {worst:.3e}"


def _level(ca, case, li, check_bwd=True, images=None):
    cfg = case["cfg"]
    N, C = cfg.levels[li]
    coords = case["coords"][li]
    feats = case["feats"][li]
    dout = case["dout"][li]
    q = case["queries"]
    dc = torch.from_numpy(coords).to(DEV)
    dq_in = torch.from_numpy(q).to(DEV)
    table = ca.knn_table(dc, cfg.G, cfg.K)
    df = feats.to(DEV)
    out = ca.knn_sample_fwd(df, dc, dq_in, table, cfg.p)
    if check_bwd:
        dF, dqg, dp = ca.knn_sample_bwd(df, dc, dq_in, table, cfg.p, dout.to(DEV))
    torch.cuda.synchronize()
    imgs = range(cfg.B) if images is None else images
    F64 = feats.double().numpy()
    dO64 = dout.double().numpy()
    dp_ref = 0.0
    for b in imgs:
        t_ref = O.knn_table(coords[b], cfg.G, cfg.K)
        t_gpu = table[b].cpu().numpy()
        diff = np.argwhere(t_gpu != t_ref)
        assert diff.size == 0, f"level {li} image {b}: {len(diff)} table mismatches, first {diff[:3].tolist()}"
        o_ref = O.knn_sample_fwd(coords[b], F64[b], q[b], t_ref, cfg.p)
        _check(f"L{li} b{b} out", out[b].double().cpu().numpy(), o_ref, _bar(feats.dtype, o_ref))
        if check_bwd:
            dF_ref, dq_ref, dp_b = O.knn_sample_bwd(coords[b], F64[b], q[b], t_ref, cfg.p, dO64[b])
            dp_ref += dp_b
            _check(f"L{li} b{b} dF", dF[b].double().cpu().numpy(), dF_ref, _bar(feats.dtype, dF_ref))
            sc = max(1.0, float(np.abs(dq_ref).max()))
            _check(f"L{li} b{b} dq", dqg[b].double().cpu().numpy(), dq_ref,
                   2e-4 * sc + 1e-3 * np.abs(dq_ref))
    if check_bwd and images is None:
        _check(f"L{li} dp", np.array([float(dp.item())]), np.array([dp_ref]),
               np.array([1e-4 * max(1.0, abs(dp_ref)) + 1e-4 * np.sqrt(cfg.B * cfg.M * cfg.K)]))
    return table, out


@pytest.mark.parametrize("li", [0, 1])
def test_tiny_fp32_levels(ca, li):
    case = make_sampler_case("knn_tiny")
    print(f"case knn_tiny level {li}", flush=True)
    _level(ca, case, li)


@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_decoder_levels_bf16(ca, li):
    case = make_sampler_case("knn_decoder", B=2)
    print(f"case knn_decoder B=2 level {li}", flush=True)
    _level(ca, case, li)


def test_decoder_full_batch_sampled_images(ca):
    """The full 32-image launch (as the benchmark runs it), images 0 and 31
    compared in full."""
    case = make_sampler_case("knn_decoder")
    for li in range(4):
        print(f"case knn_decoder B=32 level {li} images 0, 31", flush=True)
        _level(ca, case, li, images=[0, 31])


@pytest.mark.parametrize("G,K,N", [(40, 16, 300), (7, 3, 2), (64, 5, 4096), (1, 4, 9)])
def test_table_edge_shapes(ca, G, K, N):
    """G not a power of two, K = 16, fewer tokens than slots, the largest
    image, a one-cell grid; coordinates outside the grid and repeated ones."""
    rng = np.random.default_rng(G * 100 + K)
    pts = rng.uniform(-3.0, G + 2.0, size=(2, N, 2)).astype(np.float32)
    pts[:, N // 2:] = pts[:, : N - N // 2]            # repeated coordinates: distance ties
    print(f"case table G={G} K={K} N={N}", flush=True)
    table = ca.knn_table(torch.from_numpy(pts).to(DEV), G, K).cpu().numpy()
    for b in range(2):
        ref = O.knn_table(pts[b], G, K)
        assert np.array_equal(table[b], ref), f"image {b}"


@pytest.mark.parametrize("dtype,N,C,K,M", [(torch.float32, 100, 128, 16, 300),
                                           (torch.float16, 300, 64, 4, 129),
                                           (torch.bfloat16, 180, 128, 8, 1),
                                           (torch.bfloat16, 7, 256, 8, 500),
                                           (torch.float16, 150, 192, 8, 200),
                                           (torch.bfloat16, 120, 640, 4, 150),
                                           (torch.float32, 90, 768, 8, 100),
                                           (torch.float32, 60, 1024, 16, 64),
                                           (torch.bfloat16, 4096, 128, 8, 700)])
def test_small_images_all_dtypes(ca, dtype, N, C, K, M):
    """Small images in every element type: f32 / f16 / bf16, K = 4, 8, 16,
    rows of 128 to 4096 bytes, a query count that fills no whole wave, a
    single query, fewer tokens than slots.  The row widths also give every
    lane-group shape: one to four 16-byte chunks per lane, and groups where
    some lanes hold one chunk fewer than the others (C = 640 bf16: 80 chunks
    over 32 lanes).  4096 tokens: the largest image of the in-LDS lists."""
    G, p = 24, 0.9
    rng = np.random.default_rng(N * 7 + C + K)
    B = 2
    pts = rng.uniform(-0.5, G - 0.5, size=(B, N, 2)).astype(np.float32)
    q = rng.uniform(-2.0, G + 1.0, size=(B, M, 2)).astype(np.float32)
    F = torch.from_numpy(rng.standard_normal((B, N, C)).astype(np.float32)).to(dtype)
    dO = torch.from_numpy(rng.standard_normal((B, M, C)).astype(np.float32)).to(dtype)
    print(f"case few-token images dtype={dtype} N={N} C={C} K={K} M={M}", flush=True)
    dc = torch.from_numpy(pts).to(DEV)
    dq_in = torch.from_numpy(q).to(DEV)
    table = ca.knn_table(dc, G, K)
    out = ca.knn_sample_fwd(F.to(DEV), dc, dq_in, table, p)
    dF, dqg, dp = ca.knn_sample_bwd(F.to(DEV), dc, dq_in, table, p, dO.to(DEV))
    torch.cuda.synchronize()
    F64, dO64 = F.double().numpy(), dO.double().numpy()
    dp_ref = 0.0
    for b in range(B):
        t_ref = O.knn_table(pts[b], G, K)
        assert np.array_equal(table[b].cpu().numpy(), t_ref)
        o_ref = O.knn_sample_fwd(pts[b], F64[b], q[b], t_ref, p)
        _check(f"b{b} out", out[b].double().cpu().numpy(), o_ref, _bar(dtype, o_ref))
        dF_ref, dq_ref, dp_b = O.knn_sample_bwd(pts[b], F64[b], q[b], t_ref, p, dO64[b])
        dp_ref += dp_b
        _check(f"b{b} dF", dF[b].double().cpu().numpy(), dF_ref, _bar(dtype, dF_ref))
        sc = max(1.0, float(np.abs(dq_ref).max()))
        _check(f"b{b} dq", dqg[b].double().cpu().numpy(), dq_ref, 2e-4 * sc + 1e-3 * np.abs(dq_ref))
    _check("dp", np.array([float(dp.item())]), np.array([dp_ref]),
           np.array([1e-4 * max(1.0, abs(dp_ref)) + 1e-4 * np.sqrt(B * M * K)]))


def test_empty_token_set_and_far_queries(ca):
    """No tokens: zero output and zero gradients; queries far outside the
    grid use the clamped edge cells."""
    G, K, C, M = 8, 4, 16, 20
    rng = np.random.default_rng(3)
    q = rng.uniform(-40, 40, size=(1, M, 2)).astype(np.float32)
    coords0 = torch.zeros((1, 0, 2), dtype=torch.float32, device=DEV)
    table0 = ca.knn_table(coords0, G, K)
    assert (table0 == -1).all()
    f0 = torch.zeros((1, 0, C), dtype=torch.float32, device=DEV)
    out = ca.knn_sample_fwd(f0, coords0, torch.from_numpy(q).to(DEV), table0, 1.0)
    assert (out == 0).all()
    dF, dq, dp = ca.knn_sample_bwd(f0, coords0, torch.from_numpy(q).to(DEV), table0, 1.0,
                                   torch.ones((1, M, C), device=DEV))
    assert (dq == 0).all() and float(dp.item()) == 0.0
    pts = rng.uniform(0, G - 1, size=(1, 30, 2)).astype(np.float32)
    F = rng.standard_normal((1, 30, C)).astype(np.float32)
    dc = torch.from_numpy(pts).to(DEV)
    table = ca.knn_table(dc, G, K)
    out = ca.knn_sample_fwd(torch.from_numpy(F).to(DEV), dc, torch.from_numpy(q).to(DEV), table, 0.8)
    ref = O.knn_sample_fwd(pts[0], F[0].astype(np.float64), q[0], O.knn_table(pts[0], G, K), 0.8)
    _check("far queries out", out[0].double().cpu().numpy(), ref, _bar(torch.float32, ref))


def test_backward_is_deterministic(ca):
    case = make_sampler_case("knn_decoder", B=4)
    li = 3                                         # 131 tokens: long token segments
    cfg = case["cfg"]
    dc = torch.from_numpy(case["coords"][li]).to(DEV)
    dq_in = torch.from_numpy(case["queries"]).to(DEV)
    f = case["feats"][li].to(DEV)
    do = case["dout"][li].to(DEV)
    table = ca.knn_table(dc, cfg.G, cfg.K)
    r1 = ca.knn_sample_bwd(f, dc, dq_in, table, cfg.p, do)
    r2 = ca.knn_sample_bwd(f, dc, dq_in, table, cfg.p, do)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_autograd_wrapper(ca):
    case = make_sampler_case("knn_tiny")
    cfg = case["cfg"]
    dc = torch.from_numpy(case["coords"][0]).to(DEV)
    qv = torch.from_numpy(case["queries"]).to(DEV).requires_grad_(True)
    f = case["feats"][0].to(DEV).requires_grad_(True)
    table = ca.knn_table(dc, cfg.G, cfg.K)
    out = ca.knn_sample(f, dc, qv, table, cfg.p)
    out.backward(case["dout"][0].to(DEV))
    dF, dq, _ = ca.knn_sample_bwd(f.detach(), dc, qv.detach(), table, cfg.p, case["dout"][0].to(DEV))
    assert torch.equal(f.grad, dF) and torch.equal(qv.grad, dq)
