"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

from gathered_local_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cluster_attn.h")

CA_OK, CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_UNSUPPORTED, CA_ERR_WORKSPACE, CA_ERR_ALIAS = range(6)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(cluster_attn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks a signature for {n}"


def test_status_strings(lib):
    for s in range(7):
        assert lib.cluster_attn_status_string(s).startswith(b"CA_")
    assert lib.cluster_attn_version().startswith(b"clusterattn")


P = 0x10000  # fake, never-dereferenced device pointers (validation fails first)


def fwd(lib, dt=1, B=2, N=64, H=2, D=32, cs=8, nk=48, scale=0.17, ptrs=None):
    p = ptrs or [P * (i + 1) for i in range(7)]
    return lib.cluster_attn_fwd(dt, B, N, H, D, cs, nk, scale, *p, None)


def test_fwd_validation(lib):
    assert fwd(lib, dt=7) == CA_ERR_UNSUPPORTED
    assert b"dtype" in lib.cluster_attn_last_error()
    assert fwd(lib, N=-8) == CA_ERR_SHAPE
    assert fwd(lib, B=1 << 20, N=1 << 12) == CA_ERR_SHAPE          # B*N beyond int32
    assert fwd(lib, D=64) == CA_ERR_UNSUPPORTED
    assert fwd(lib, cs=4, nk=24) == CA_ERR_UNSUPPORTED
    assert fwd(lib, nk=50) == CA_ERR_UNSUPPORTED
    assert fwd(lib, nk=72) == CA_ERR_UNSUPPORTED
    assert fwd(lib, H=0) == CA_ERR_SHAPE
    assert fwd(lib, B=-1) == CA_ERR_SHAPE
    assert fwd(lib, scale=float("nan")) == CA_ERR_SHAPE
    assert fwd(lib, ptrs=[P, 2 * P, 3 * P, None, 5 * P, 6 * P, 7 * P]) == CA_ERR_NULL
    # empty problems are valid no-ops, even with NULL pointers
    assert fwd(lib, B=0, ptrs=[None] * 7) == CA_OK
    assert fwd(lib, N=0, ptrs=[None] * 7) == CA_OK


def test_fwd_alias_detection(lib):
    tb = 2 * 64 * 2 * 32 * 2
    base = 1 << 30
    q, k, v = base, base + tb, base + 2 * tb
    qi, ki = base + 3 * tb, base + 4 * tb
    o = base + 10 * tb
    lse = base + 20 * tb
    assert fwd(lib, ptrs=[q, k, v, qi, ki, q + 64, lse]) == CA_ERR_ALIAS        # o over q
    assert fwd(lib, ptrs=[q, k, v, qi, ki, o, o + 128]) == CA_ERR_ALIAS         # lse over o
    assert fwd(lib, ptrs=[q, k, v, qi, ki, o, ki]) == CA_ERR_ALIAS              # lse over key_idx


def bwd(lib, ws_bytes=1 << 40, ws=P * 40, dt=1, B=2, N=64, H=2, nk=48, ptrs=None):
    p = ptrs or [P * (i + 1) for i in range(11)]
    return lib.cluster_attn_bwd(dt, B, N, H, 32, 8, nk, 0.17, *p, ws, ws_bytes, None)


def test_bwd_validation_and_workspace(lib):
    need = lib.cluster_attn_bwd_workspace(1, 2, 64, 2, 32, 8, 48)
    assert need > 0
    # a partial last cluster (60 = 7*8 + 4) is a valid size
    assert lib.cluster_attn_bwd_workspace(1, 2, 60, 2, 32, 8, 48) > 0
    assert lib.cluster_attn_bwd_workspace(1, 2, -4, 2, 32, 8, 48) == 0
    assert lib.cluster_attn_bwd_workspace(9, 2, 64, 2, 32, 8, 48) == 0
    assert bwd(lib, ws_bytes=need - 1) == CA_ERR_WORKSPACE
    assert bwd(lib, ws=None) == CA_ERR_NULL
    assert bwd(lib, dt=3) == CA_ERR_UNSUPPORTED
    assert bwd(lib, N=-1) == CA_ERR_SHAPE
    # dk overlapping the workspace
    p = [P * (i + 1) for i in range(11)]
    assert bwd(lib, ws=p[9] + 8, ptrs=p) == CA_ERR_ALIAS
    assert bwd(lib, B=0, ptrs=[None] * 11, ws=None) == CA_OK


def test_workspace_grows_with_problem(lib):
    a = lib.cluster_attn_bwd_workspace(1, 32, 2048, 4, 32, 8, 48)
    b = lib.cluster_attn_bwd_workspace(1, 64, 2048, 4, 32, 8, 48)
    assert b > a > 0
    # An image of at most 4096 tokens is built in one workgroup's LDS.
    assert lib.cluster_attn_build_neighbors_workspace(4, 2048, 8, 6) == 0
    assert lib.cluster_attn_build_neighbors_workspace(4, 4096, 8, 6) == 0
    assert lib.cluster_attn_build_neighbors_workspace(4, 65536, 8, 6) > \
        lib.cluster_attn_build_neighbors_workspace(4, 8192, 8, 6) > 0


def test_build_validation(lib):
    def build(B=2, N=64, G=32, cs=8, k=6, ws_bytes=1 << 30, ptrs=None, ws=P * 9):
        p = ptrs or [P, 2 * P, 3 * P, 4 * P]
        return lib.cluster_attn_build_neighbors(p[0], B, N, G, cs, k, p[1], p[2], p[3], ws,
                                                ws_bytes, None)
    assert build(N=(1 << 22) + 8) == CA_ERR_SHAPE                   # beyond 2^22 per image
    assert build(N=-3) == CA_ERR_SHAPE
    assert build(cs=16) == CA_ERR_UNSUPPORTED
    assert build(k=0) == CA_ERR_UNSUPPORTED
    assert build(k=9) == CA_ERR_UNSUPPORTED
    assert build(G=0) == CA_ERR_SHAPE
    assert build(G=70000) == CA_ERR_SHAPE
    assert build(ptrs=[P, None, 3 * P, 4 * P]) == CA_ERR_NULL
    assert build(N=8192, ws_bytes=16) == CA_ERR_WORKSPACE
    assert build(N=8192, ws=None) == CA_ERR_NULL
    assert build(ptrs=[P, 2 * P, 2 * P + 4, 4 * P]) == CA_ERR_ALIAS
    assert build(B=0, ptrs=[None] * 4, ws=None) == CA_OK


def test_varlen_validation(lib):
    def build(B=3, T=100, Ct=14, max_n=50, G=32, k=6, ws_bytes=1 << 30, ptrs=None, ws=P * 9):
        p = ptrs or [P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P]
        return lib.cluster_attn_build_neighbors_varlen(p[0], B, T, Ct, max_n, p[1], p[2], G, 8, k,
                                                       p[3], p[4], p[5], ws, ws_bytes, None)
    assert build(max_n=101) == CA_ERR_SHAPE                         # an image above T
    assert build(Ct=12) == CA_ERR_SHAPE                             # fewer than ceil(T/8)
    assert build(Ct=101) == CA_ERR_SHAPE                            # more clusters than tokens
    assert build(k=9) == CA_ERR_UNSUPPORTED
    assert build(ptrs=[P, None, 3 * P, 4 * P, 5 * P, 6 * P]) == CA_ERR_NULL
    assert build(ptrs=[P, 2 * P, 3 * P, 4 * P, 4 * P + 8, 6 * P]) == CA_ERR_ALIAS
    assert build(max_n=5000, T=6000, Ct=760, ws_bytes=8) == CA_ERR_WORKSPACE
    assert build(B=0, T=0, Ct=0, max_n=0, ptrs=[None] * 6, ws=None) == CA_OK
    assert lib.cluster_attn_build_neighbors_varlen_workspace(3, 100, 14, 50, 8, 6) == 0
    assert lib.cluster_attn_build_neighbors_varlen_workspace(3, 6000, 760, 3000, 8, 6) == 0
    assert lib.cluster_attn_build_neighbors_varlen_workspace(3, 6000, 760, 5000, 8, 6) > 0
    assert lib.cluster_attn_build_neighbors_varlen_workspace(3, 100, 14, 101, 8, 6) == 0

    p7 = [P * (i + 1) for i in range(7)]
    f = lambda T=100, Ct=14, nk=48, ptrs=p7: lib.cluster_attn_fwd_varlen(
        1, T, Ct, 2, 32, 8, nk, 0.17, *ptrs, None)
    assert f(Ct=12) == CA_ERR_SHAPE
    assert f(Ct=101) == CA_ERR_SHAPE
    assert f(nk=50) == CA_ERR_UNSUPPORTED
    assert f(ptrs=[P, 2 * P, None, 4 * P, 5 * P, 6 * P, 7 * P]) == CA_ERR_NULL
    assert f(T=0, Ct=0, ptrs=[None] * 7) == CA_OK
    need = lib.cluster_attn_bwd_varlen_workspace(1, 100, 14, 2, 32, 8, 48)
    assert need > 0 and lib.cluster_attn_bwd_varlen_workspace(1, 100, 12, 2, 32, 8, 48) == 0
    p11 = [P * (i + 1) for i in range(11)]
    assert lib.cluster_attn_bwd_varlen(1, 100, 14, 2, 32, 8, 48, 0.17, *p11, P * 40, need - 1,
                                       None) == CA_ERR_WORKSPACE


def test_3d_build_validation(lib):
    def build(B=2, N=64, G=32, k=6, ptrs=None, ws_bytes=1 << 30, ws=P * 9):
        p = ptrs or [P, 2 * P, 3 * P, 4 * P]
        return lib.cluster_attn_build_neighbors_3d(p[0], B, N, G, 8, k, p[1], p[2], p[3], ws,
                                                   ws_bytes, None)
    assert build(G=16385) == CA_ERR_SHAPE            # 14-bit axes: G up to 2^14
    assert build(G=0) == CA_ERR_SHAPE
    assert build(k=9) == CA_ERR_UNSUPPORTED
    assert build(N=8192, ws_bytes=16) == CA_ERR_WORKSPACE
    assert build(ptrs=[P, None, 3 * P, 4 * P]) == CA_ERR_NULL
    assert build(ptrs=[P + 8, 2 * P, 3 * P, 4 * P], N=(P // 12)) == CA_ERR_ALIAS   # 12 B per token
    assert build(B=0, ptrs=[None] * 4, ws=None) == CA_OK
    p6 = [P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P]
    assert lib.cluster_attn_build_neighbors_varlen_3d(p6[0], 3, 100, 12, 50, p6[1], p6[2], 16, 8, 6,
                                                      p6[3], p6[4], p6[5], P * 9, 1 << 20,
                                                      None) == CA_ERR_SHAPE


def test_plan_validation(lib):
    assert lib.cluster_attn_bwd_plan_workspace(2, 64, 8, 8, 48) > 0
    assert lib.cluster_attn_bwd_plan_workspace(2, 64, 9, 8, 48) == 0        # C != ceil(N/8), B > 1
    assert lib.cluster_attn_bwd_plan_workspace(1, 100, 20, 8, 48) > 0      # packed: 13 <= C <= N
    assert lib.cluster_attn_bwd_plan_workspace(1, 100, 101, 8, 48) == 0
    need = lib.cluster_attn_bwd_plan_workspace(2, 64, 8, 8, 48)
    assert lib.cluster_attn_bwd_plan(2, 64, 8, 8, 48, P, 2 * P, 3 * P, need - 1, None) == CA_ERR_WORKSPACE
    assert lib.cluster_attn_bwd_plan(2, 64, 8, 8, 48, P, None, 3 * P, need, None) == CA_ERR_NULL
    assert lib.cluster_attn_bwd_plan(2, 64, 8, 8, 48, P, 2 * P, 2 * P + 4, need, None) == CA_ERR_ALIAS
    assert lib.cluster_attn_bwd_plan(0, 64, 8, 8, 48, None, None, None, 0, None) == CA_OK
    p11 = [P * (i + 1) for i in range(11)]
    call = lambda plan, pb, ws, wb: lib.cluster_attn_bwd_planned(
        1, 2, 64, 8, 2, 32, 8, 48, 0.17, *p11[:8], plan, pb, *p11[8:], ws, wb, None)
    wneed = lib.cluster_attn_bwd_planned_workspace(1, 2, 64, 2, 32)
    assert 0 < wneed < lib.cluster_attn_bwd_workspace(1, 2, 64, 2, 32, 8, 48)
    assert call(None, 0, P * 40, wneed) == CA_ERR_NULL
    assert call(P * 30, need - 1, P * 40, wneed) == CA_ERR_WORKSPACE
    assert call(P * 30, need, P * 40, wneed - 1) == CA_ERR_WORKSPACE
    assert call(p11[9], need, P * 40, wneed) == CA_ERR_ALIAS              # plan over dk (an input over an output)


def test_missing_library_raises(tmp_path):
    with pytest.raises(_lib.LibraryMissing):
        _lib.load(str(tmp_path / "nope.so"))


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "gathered_local_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("no oracle", ""), f


def knn_fwd(lib, dt=1, B=2, N=100, M=50, C=128, G=16, K=8, p=1.0, ptrs=None):
    ps = ptrs or [P * (i + 1) for i in range(5)]
    return lib.cluster_attn_knn_sample_fwd(dt, B, N, M, C, G, K, p, *ps, None)


def test_knn_validation(lib):
    # table build limits
    t = lib.cluster_attn_knn_table
    assert t(P, 2, 100, 2049, 8, 2 * P, None, 0, None) == CA_ERR_UNSUPPORTED   # G > 2048
    assert t(P, 2, (1 << 24) + 1, 64, 8, 2 * P, None, 0, None) == CA_ERR_SHAPE
    assert t(P, 2, 100, 64, 17, 2 * P, None, 0, None) == CA_ERR_UNSUPPORTED    # K > 16
    assert t(P, 2, 100, 0, 8, 2 * P, None, 0, None) == CA_ERR_UNSUPPORTED
    assert t(None, 2, 100, 64, 8, 2 * P, None, 0, None) == CA_ERR_NULL
    assert t(P, -1, 100, 64, 8, 2 * P, None, 0, None) == CA_ERR_SHAPE
    assert t(None, 0, 100, 64, 8, None, None, 0, None) == CA_OK                # empty batch
    assert t(P, 2, 100, 16, 8, P + 8, None, 0, None) == CA_ERR_ALIAS           # table over coords
    # images above 4096 tokens are bucketed in a workspace
    assert lib.cluster_attn_knn_table_workspace(2, 4096, 64) == 0
    need = lib.cluster_attn_knn_table_workspace(2, 32768, 256)
    assert need >= 2 * 32768 * 12
    assert lib.cluster_attn_knn_table_workspace(2, 32768, 4096) == 0         # invalid G
    assert t(P, 2, 32768, 256, 8, 2 * P, None, need, None) == CA_ERR_NULL
    assert t(P, 2, 32768, 256, 8, 2 * P, 8 * P, need - 1, None) == CA_ERR_WORKSPACE
    assert t(P, 2, 32768, 256, 8, 2 * P, P + 64, need, None) == CA_ERR_ALIAS  # ws over coords
    # sampler
    assert knn_fwd(lib, dt=5) == CA_ERR_UNSUPPORTED
    assert knn_fwd(lib, C=12) == CA_ERR_UNSUPPORTED
    assert knn_fwd(lib, C=2048) == CA_ERR_UNSUPPORTED
    assert knn_fwd(lib, K=0) == CA_ERR_UNSUPPORTED
    assert knn_fwd(lib, G=0) == CA_ERR_SHAPE
    assert knn_fwd(lib, M=-3) == CA_ERR_SHAPE
    assert knn_fwd(lib, p=float("inf")) == CA_ERR_SHAPE
    assert knn_fwd(lib, ptrs=[P, 2 * P, None, 4 * P, 5 * P]) == CA_ERR_NULL
    assert knn_fwd(lib, M=0, ptrs=[None] * 5) == CA_OK
    base = 1 << 30
    fb = 2 * 100 * 128 * 2
    ptrs = [base, base + 4096, base + 4096 + fb, base + 2 * fb, base + 4096 + 16]   # out over feats
    assert knn_fwd(lib, ptrs=ptrs) == CA_ERR_ALIAS
    # backward: workspace size and NULL dp
    need = lib.cluster_attn_knn_sample_bwd_workspace(2, 100, 50, 8)
    assert need > 2 * 50 * 8 * 12
    assert lib.cluster_attn_knn_sample_bwd_workspace(2, 100, 50, 17) == 0
    ten = [P * (i + 1) for i in range(7)]   # coords, feats, queries, table, dout, dfeats, dq
    b = lib.cluster_attn_knn_sample_bwd
    assert b(1, 2, 100, 50, 128, 16, 8, 1.0, *ten, None, P * 50, need, None) == CA_ERR_NULL
    assert b(1, 2, 100, 50, 128, 16, 8, 1.0, *ten, P * 60, None, need, None) == CA_ERR_NULL
    assert b(1, 2, 100, 50, 128, 16, 8, 1.0, *ten, P * 60, P * 50, need - 1, None) == CA_ERR_WORKSPACE


def test_merge_validation(lib):
    pl = lib.cluster_attn_merge_plan
    ptr = [P * (i + 1) for i in range(6)]
    assert pl(*ptr[:2], 2, (1 << 24) + 1, 100, 64, *ptr[2:], None, 0, None) == CA_ERR_SHAPE
    assert pl(*ptr[:2], 2, 100, 0, 64, *ptr[2:], None, 0, None) == CA_ERR_SHAPE     # k < 1
    assert pl(*ptr[:2], 2, 100, 101, 64, *ptr[2:], None, 0, None) == CA_ERR_SHAPE   # k > N
    assert pl(*ptr[:2], 2, 100, 40, 0, *ptr[2:], None, 0, None) == CA_ERR_SHAPE     # grid side
    assert pl(None, P, 2, 100, 40, 64, *ptr[2:], None, 0, None) == CA_ERR_NULL
    assert pl(None, None, 0, 100, 40, 64, None, None, None, None, None, 0, None) == CA_OK
    # images above 4096 tokens are planned in a workspace
    assert lib.cluster_attn_merge_plan_workspace(2, 4096, 1000) == 0
    need = lib.cluster_attn_merge_plan_workspace(2, 65536, 26214)
    assert need >= 2 * (65536 * 12 + 26214 * 16)
    assert lib.cluster_attn_merge_plan_workspace(2, 100, 101) == 0                # k > N
    big = [P * 64 * (i + 1) for i in range(6)]
    assert pl(*big[:2], 2, 65536, 26214, 256, *big[2:], None, need, None) == CA_ERR_NULL
    assert pl(*big[:2], 2, 65536, 26214, 256, *big[2:], P * 2048, need - 1, None) == CA_ERR_WORKSPACE
    fw = lib.cluster_attn_merge_fwd
    t = [P * (i + 1) for i in range(7)]
    assert fw(9, 2, 100, 40, 64, *t, None) == CA_ERR_UNSUPPORTED
    assert fw(1, 2, 100, 40, 60, *t, None) == CA_ERR_UNSUPPORTED                  # C % 8
    assert fw(1, 2, 100, 40, 64, *t[:6], None, None) == CA_ERR_NULL
    bw = lib.cluster_attn_merge_bwd
    u = [P * (i + 1) for i in range(10)]
    assert bw(1, 2, 100, 140, 64, *u, None) == CA_ERR_SHAPE
    assert bw(1, 2, 100, 40, 64, *u[:9], None, None) == CA_ERR_NULL
