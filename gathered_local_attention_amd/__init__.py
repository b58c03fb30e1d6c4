"""Local cluster attention over off-grid tokens on MI355X (gfx950).

Thin Python binding over the C ABI of ``libclusterattn.so`` (declared in
``include/cluster_attn.h``).  Every step of the computation runs in the HIP
kernels; this module only checks tensor properties, allocates outputs with
torch and passes raw device pointers plus the current HIP stream.  There is
no CPU fallback: if the library is missing, the calls raise.

Functions
---------
build_neighbors(coords, grid_side, cs=8, k=6) -> (perm, nbr, key_idx)   (2D or 3D)
fwd(q, k, v, q_idx, key_idx, scale=None) -> (o, lse)
bwd(q, k, v, o, do, lse, q_idx, key_idx, scale=None, plan=None) -> (dq, dk, dv)
bwd_plan(q_idx, key_idx, N) -> plan   (transposed lists, reusable across backward calls)
check_lists(q_idx, key_idx, N)   (host-side index validation; fwd/bwd take check=True)
cluster_attention(q, k, v, q_idx, key_idx, scale=None) -> o   (autograd)
build_neighbors_varlen(coords, lengths, grid_side, cs=8, k=6)
    -> (q_idx, nbr, key_idx, tok_off, clu_off)        (packed batches)
fwd_varlen(q, k, v, q_idx, key_idx, scale=None) -> (o, lse)
bwd_varlen(q, k, v, o, do, lse, q_idx, key_idx, scale=None) -> (dq, dk, dv)
knn_table(coords, grid_side, K, workspace=None) -> table
knn_sample_fwd(feats, coords, queries, table, p) -> out
knn_sample_bwd(feats, coords, queries, table, p, dout) -> (dfeats, dq, dp)
knn_sample(feats, coords, queries, table, p) -> out   (autograd: feats, queries)
merge_plan(coords, scores, k, grid_side, workspace=None) -> (anchors, assign, members, offsets)
merge_fwd(feats, coords, scores, members, offsets, k) -> (out_feats, out_coords)
merge_bwd(feats, coords, scores, members, offsets, dout_feats, dout_coords)
    -> (dfeats, dcoords, dscores)
"""

from __future__ import annotations

import math

import torch

from . import _lib

__all__ = [
    "build_neighbors",
    "check_lists",
    "device_copy",
    "fwd",
    "bwd",
    "cluster_attention",
    "bwd_plan",
    "bwd_plan_varlen",
    "bwd_planned_noalloc",
    "build_neighbors_varlen",
    "fwd_varlen",
    "bwd_varlen",
    "varlen_offsets",
    "bwd_workspace_bytes",
    "build_workspace_bytes",
    "knn_table",
    "knn_table_workspace_bytes",
    "knn_sample_fwd",
    "knn_sample_bwd",
    "knn_sample",
    "knn_bwd_workspace_bytes",
    "merge_plan",
    "merge_plan_workspace_bytes",
    "merge_fwd",
    "merge_bwd",
    "ClusterAttnError",
    "CA_OK",
]

CA_OK = 0
_DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


class ClusterAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        msg = lib.cluster_attn_status_string(status).decode()
        detail = lib.cluster_attn_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))
        self.status = status


def _check(status: int, where: str):
    if status != CA_OK:
        raise ClusterAttnError(status, where)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def device_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """dst[:] = src with the library's plain copy kernel (a bandwidth probe
    for measurement; both contiguous device tensors of equal byte size)."""
    if dst.numel() * dst.element_size() != src.numel() * src.element_size():
        raise ValueError("dst and src differ in size")
    _check(_lib.load().cluster_attn_device_copy(_dev(dst, "dst"), _dev(src, "src"),
                                                src.numel() * src.element_size(), _stream(src)),
           "cluster_attn_device_copy")


def build_workspace_bytes(B: int, N: int, cs: int = 8, k: int = 6) -> int:
    return int(_lib.load().cluster_attn_build_neighbors_workspace(B, N, cs, k))


def bwd_workspace_bytes(dtype: torch.dtype, B: int, N: int, H: int, D: int = 32, cs: int = 8,
                        nk: int = 48) -> int:
    return int(_lib.load().cluster_attn_bwd_workspace(_DT[dtype], B, N, H, D, cs, nk))


def build_neighbors(coords: torch.Tensor, grid_side: int, cs: int = 8, k: int = 6,
                    workspace: torch.Tensor | None = None):
    """Morton-order balanced clusters and nearest-cluster key lists.

    coords: [B, N, 2] float32 device tensor (x = column, y = row), or
    [B, N, 3] for 3D tokens (z = slice; 14-bit fixed point per axis).
    Returns perm [B, C*cs] (== q_idx [B, C, cs] as a view, C = ceil(N/cs);
    -1 after the members of a partial last cluster), nbr [B, C, k] and
    key_idx [B, C, cs*k], all int32."""
    lib = _lib.load()
    B, N, dims = coords.shape
    if dims not in (2, 3):
        raise ValueError("coords must be [B, N, 2] or [B, N, 3]")
    _dev(coords, "coords", torch.float32)
    C = -(-N // cs) if cs else 0
    perm = torch.empty((B, C * cs), dtype=torch.int32, device=coords.device)
    nbr = torch.empty((B, C, k), dtype=torch.int32, device=coords.device)
    key_idx = torch.empty((B, C, cs * k), dtype=torch.int32, device=coords.device)
    need = lib.cluster_attn_build_neighbors_workspace(B, N, cs, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=coords.device)
    fn = lib.cluster_attn_build_neighbors if dims == 2 else lib.cluster_attn_build_neighbors_3d
    _check(fn(coords.data_ptr(), B, N, int(grid_side), cs, k, perm.data_ptr(), nbr.data_ptr(),
              key_idx.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(coords)),
           "cluster_attn_build_neighbors" + ("" if dims == 2 else "_3d"))
    return perm, nbr, key_idx


def _shapes(q, q_idx, key_idx, cs: int = 8):
    """Sizes of a batched call, with the index lists checked against them:
    q_idx [B, C, cs] (or its [B, C*cs] flat form) and key_idx [B, C, nk]
    with C = ceil(N / cs).  The C entry points read B*C*cs and B*C*nk
    indices, so a mismatch must be caught here, before any launch."""
    if q.dim() != 4:
        raise ValueError("q/k/v must be [B, N, H, D]")
    B, N, H, D = q.shape
    C = -(-N // cs)
    if q_idx.dim() == 2:
        if q_idx.shape != (B, C * cs):
            raise ValueError(f"q_idx must be [B, C*cs] = [{B}, {C * cs}], got {list(q_idx.shape)}")
        q_idx = q_idx.view(B, C, cs)
    if q_idx.shape != (B, C, cs):
        raise ValueError(f"q_idx must be [B, C, cs] = [{B}, {C}, {cs}], got {list(q_idx.shape)}")
    if key_idx.dim() != 3 or key_idx.shape[:2] != (B, C):
        raise ValueError(f"key_idx must be [B, C, nk] = [{B}, {C}, nk], got {list(key_idx.shape)}")
    nk = key_idx.shape[-1]
    return B, N, H, D, cs, nk, q_idx


def _check_lse(lse, B, N, H):
    if lse.shape != (B, N, H):
        raise ValueError(f"lse must be [B, N, H] = [{B}, {N}, {H}], got {list(lse.shape)}")


def check_lists(q_idx: torch.Tensor, key_idx: torch.Tensor, N: int) -> None:
    """Validate index lists on the host (``cluster_attn_check_lists``):
    q_idx [B, C, cs] / [B, C*cs] (or [Ct, cs] for a packed batch of N = T
    tokens), key_idx [B, C, nk] / [Ct, nk].  Copies the lists to host memory
    (a synchronisation for device tensors) and raises ClusterAttnError with
    the first offending position if a value is out of range or q_idx does
    not partition the tokens.  The kernels themselves never check."""
    lib = _lib.load()
    qh = q_idx.detach().to("cpu", torch.int32).contiguous()
    kh = key_idx.detach().to("cpu", torch.int32).contiguous()
    if kh.dim() == 3:
        B, C, nk = kh.shape
        cs = qh.numel() // max(1, B * C) if B * C else 8
    elif kh.dim() == 2:
        B, (C, nk) = 1, kh.shape
        cs = qh.shape[-1]
    else:
        raise ValueError("key_idx must be [B, C, nk] or [Ct, nk]")
    if qh.numel() != B * C * cs:
        raise ValueError("q_idx and key_idx disagree on the number of clusters")
    _check(lib.cluster_attn_check_lists(B, int(N), C, cs, nk, qh.data_ptr(), kh.data_ptr()),
           "cluster_attn_check_lists")


def fwd(q, k, v, q_idx, key_idx, scale: float | None = None, check: bool = False):
    """Forward: returns O [B, N, H, D] (dtype of q) and LSE [B, N, H] f32.
    ``check`` validates the index lists on the host first
    (:func:`check_lists`; synchronises)."""
    lib = _lib.load()
    B, N, H, D, cs, nk, q_idx = _shapes(q, q_idx, key_idx)
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t, n in ((k, "k"), (v, "v")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q in shape and dtype")
    if check:
        check_lists(q_idx, key_idx, N)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, N, H), dtype=torch.float32, device=q.device)
    _check(lib.cluster_attn_fwd(
        _DT[q.dtype], B, N, H, D, cs, nk, scale, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
        _dev(q_idx, "q_idx", torch.int32), _dev(key_idx, "key_idx", torch.int32),
        o.data_ptr(), lse.data_ptr(), _stream(q)), "cluster_attn_fwd")
    return o, lse


def bwd_plan(q_idx: torch.Tensor, key_idx: torch.Tensor, N: int) -> torch.Tensor:
    """Transposed slot lists of the backward, built once for lists that
    several backward calls share: q_idx [B, C, cs] (or [B, C*cs]) and
    key_idx [B, C, nk] of B images of N tokens, or q_idx [Ct, cs] and
    key_idx [Ct, nk] of a packed batch of N = T tokens.  Returns a uint8
    device tensor to pass as ``plan=`` to :func:`bwd` / :func:`bwd_varlen`."""
    lib = _lib.load()
    if key_idx.dim() == 3:
        B, C, nk = key_idx.shape
        cs = 8
        if C != -(-int(N) // cs):
            raise ValueError(f"key_idx has {C} clusters per image, N={N} needs {-(-int(N) // cs)}")
    elif key_idx.dim() == 2:
        B, (C, nk) = 1, key_idx.shape
        cs = q_idx.shape[-1]
        if C < -(-int(N) // cs) or C > int(N):
            raise ValueError(f"a packed batch of {N} tokens cannot have {C} clusters")
    else:
        raise ValueError("key_idx must be [B, C, nk] or [Ct, nk]")
    if q_idx.numel() != B * C * cs:
        raise ValueError(f"q_idx must hold B*C*cs = {B * C * cs} indices, has {q_idx.numel()}")
    need = lib.cluster_attn_bwd_plan_workspace(B, int(N), C, cs, nk)
    plan = torch.empty(max(need, 1), dtype=torch.uint8, device=key_idx.device)
    _check(lib.cluster_attn_bwd_plan(B, int(N), C, cs, nk, _dev(q_idx, "q_idx", torch.int32),
                                     _dev(key_idx, "key_idx", torch.int32), plan.data_ptr(),
                                     plan.numel(), _stream(key_idx)), "cluster_attn_bwd_plan")
    return plan


def bwd_plan_varlen(q_idx: torch.Tensor, key_idx: torch.Tensor, lengths, offsets=None) -> torch.Tensor:
    """The plan of a packed batch (q_idx [Ct, cs], key_idx [Ct, nk] from
    :func:`build_neighbors_varlen`), built one image at a time; ``offsets``
    = the (tok_off, clu_off) device pair that call returned (else uploaded
    from ``lengths``).  Pass the result as ``plan=`` to :func:`bwd_varlen`."""
    lib = _lib.load()
    Ct, cs = q_idx.shape
    nk = key_idx.shape[1]
    tok, clu = varlen_offsets(lengths, cs)
    B, T = len(tok) - 1, tok[-1]
    max_n = max((tok[b + 1] - tok[b] for b in range(B)), default=0)
    if offsets is None:
        offsets = (torch.tensor(tok, dtype=torch.int32).to(q_idx.device),
                   torch.tensor(clu, dtype=torch.int32).to(q_idx.device))
    need = lib.cluster_attn_bwd_plan_workspace(1, T, Ct, cs, nk)
    plan = torch.empty(max(need, 1), dtype=torch.uint8, device=q_idx.device)
    _check(lib.cluster_attn_bwd_plan_varlen(
        B, T, Ct, max_n, _dev(offsets[0], "tok_off", torch.int32),
        _dev(offsets[1], "clu_off", torch.int32), cs, nk, _dev(q_idx, "q_idx", torch.int32),
        _dev(key_idx, "key_idx", torch.int32), plan.data_ptr(), plan.numel(), _stream(q_idx)),
        "cluster_attn_bwd_plan_varlen")
    return plan


def _bwd_planned(lib, dt, B, N, C, H, D, cs, nk, scale, q, k, v, o, do, lse, q_idx, key_idx,
                 plan, workspace):
    need = lib.cluster_attn_bwd_planned_workspace(dt, B, N, H, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _check(lib.cluster_attn_bwd_planned(
        dt, B, N, C, H, D, cs, nk, scale, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
        _dev(do, "do"), _dev(lse, "lse", torch.float32), _dev(q_idx, "q_idx", torch.int32),
        _dev(key_idx, "key_idx", torch.int32), _dev(plan, "plan"), plan.numel(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(q)),
        "cluster_attn_bwd_planned")
    return dq, dk, dv


def bwd_planned_noalloc(q, k, v, o, do, lse, q_idx, key_idx, plan: torch.Tensor,
                        scale: float | None = None, out=None):
    """The planned backward with no workspace: the library keeps the
    per-call LSE/Delta pairs in its own per-GPU scratch (B*N*H at most
    ``_lib.load().cluster_attn_bwd_planned_noalloc_max_rows()``).  ``out``:
    optional (dq, dk, dv) tensors to write, so that nothing is allocated
    here either.  Calls that overlap on one GPU share the scratch and must
    be serialised by the caller."""
    lib = _lib.load()
    B, N, H, D, cs, nk, q_idx = _shapes(q, q_idx, key_idx)
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q in shape and dtype")
    _check_lse(lse, B, N, H)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    for t in out:
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("out tensors must match q in shape and dtype")
    dq, dk, dv = out
    _check(lib.cluster_attn_bwd_planned_noalloc(
        _DT[q.dtype], B, N, q_idx.shape[1], H, D, cs, nk, scale, _dev(q, "q"), _dev(k, "k"),
        _dev(v, "v"), _dev(o, "o"), _dev(do, "do"), _dev(lse, "lse", torch.float32),
        _dev(q_idx, "q_idx", torch.int32), _dev(key_idx, "key_idx", torch.int32),
        _dev(plan, "plan"), plan.numel(), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"),
        _stream(q)), "cluster_attn_bwd_planned_noalloc")
    return dq, dk, dv


def bwd(q, k, v, o, do, lse, q_idx, key_idx, scale: float | None = None,
        workspace: torch.Tensor | None = None, plan: torch.Tensor | None = None,
        check: bool = False):
    """Backward: returns dQ, dK, dV (dtype of q).  ``plan`` (from
    :func:`bwd_plan` on the same lists) skips rebuilding the transposed
    lists; the result is the same bit for bit.  ``check`` validates the
    index lists on the host first (:func:`check_lists`; synchronises)."""
    lib = _lib.load()
    B, N, H, D, cs, nk, q_idx = _shapes(q, q_idx, key_idx)
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q in shape and dtype")
    _check_lse(lse, B, N, H)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dt = _DT[q.dtype]
    if check:
        check_lists(q_idx, key_idx, N)
    if plan is not None:
        return _bwd_planned(lib, dt, B, N, q_idx.shape[1], H, D, cs, nk, scale, q, k, v, o, do,
                            lse, q_idx, key_idx, plan, workspace)
    need = lib.cluster_attn_bwd_workspace(dt, B, N, H, D, cs, nk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _check(lib.cluster_attn_bwd(
        dt, B, N, H, D, cs, nk, scale, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
        _dev(do, "do"), _dev(lse, "lse", torch.float32), _dev(q_idx, "q_idx", torch.int32),
        _dev(key_idx, "key_idx", torch.int32), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(q)), "cluster_attn_bwd")
    return dq, dk, dv


class _ClusterAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, q_idx, key_idx, scale):
        o, lse = fwd(q, k, v, q_idx, key_idx, scale)
        ctx.save_for_backward(q, k, v, o, lse, q_idx, key_idx)
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, q_idx, key_idx = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, do.contiguous(), lse, q_idx, key_idx, ctx.scale)
        return dq, dk, dv, None, None, None


def cluster_attention(q, k, v, q_idx, key_idx, scale: float | None = None):
    """Autograd-aware local cluster attention (index lists are constants)."""
    return _ClusterAttention.apply(q, k, v, q_idx, key_idx, scale)


# ---------------------------------------------------------------------------
# Packed batches of images of different sizes
# ---------------------------------------------------------------------------

def varlen_offsets(lengths, cs: int = 8):
    """Host-side token and cluster offsets [B+1] (lists of ints) of a packed
    batch with the given per-image token counts."""
    tok, clu = [0], [0]
    for n in lengths:
        n = int(n)
        if n < 0:
            raise ValueError("negative image size")
        tok.append(tok[-1] + n)
        clu.append(clu[-1] + (-(-n // cs)))
    return tok, clu


def build_neighbors_varlen(coords: torch.Tensor, lengths, grid_side: int, cs: int = 8, k: int = 6,
                           workspace: torch.Tensor | None = None, offsets=None):
    """Neighbour lists of a packed batch: coords [T, 2] float32 (device;
    [T, 3] for 3D tokens) holds the images one after another, image b
    having lengths[b] tokens.
    Returns q_idx [Ct, cs], nbr [Ct, k], key_idx [Ct, cs*k] (int32,
    batch-global ids, -1 padding) and the device offsets tok_off, clu_off
    [B+1] int32.  ``offsets`` may pass that pair from an earlier call with
    the same lengths (no host-to-device copy then)."""
    lib = _lib.load()
    if coords.dim() != 2 or coords.shape[1] not in (2, 3):
        raise ValueError("coords must be [T, 2] or [T, 3]")
    dims = coords.shape[1]
    _dev(coords, "coords", torch.float32)
    tok, clu = varlen_offsets(lengths, cs)
    B, T, Ct = len(tok) - 1, tok[-1], clu[-1]
    if T != coords.shape[0]:
        raise ValueError(f"lengths sum to {T}, coords has {coords.shape[0]} rows")
    max_n = max((tok[b + 1] - tok[b] for b in range(B)), default=0)
    dev = coords.device
    if offsets is None:
        tok_off = torch.tensor(tok, dtype=torch.int32).to(dev)
        clu_off = torch.tensor(clu, dtype=torch.int32).to(dev)
    else:
        tok_off, clu_off = offsets
        if tok_off.numel() != B + 1 or clu_off.numel() != B + 1:
            raise ValueError("offsets do not match lengths")
        _dev(tok_off, "tok_off", torch.int32)
        _dev(clu_off, "clu_off", torch.int32)
    q_idx = torch.empty((Ct, cs), dtype=torch.int32, device=dev)
    nbr = torch.empty((Ct, k), dtype=torch.int32, device=dev)
    key_idx = torch.empty((Ct, cs * k), dtype=torch.int32, device=dev)
    need = lib.cluster_attn_build_neighbors_varlen_workspace(B, T, Ct, max_n, cs, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    fn = (lib.cluster_attn_build_neighbors_varlen if dims == 2
          else lib.cluster_attn_build_neighbors_varlen_3d)
    _check(fn(coords.data_ptr(), B, T, Ct, max_n, tok_off.data_ptr(), clu_off.data_ptr(),
              int(grid_side), cs, k, q_idx.data_ptr(), nbr.data_ptr(), key_idx.data_ptr(),
              workspace.data_ptr(), workspace.numel(), _stream(coords)),
           "cluster_attn_build_neighbors_varlen" + ("" if dims == 2 else "_3d"))
    return q_idx, nbr, key_idx, tok_off, clu_off


def _varlen_shapes(q, q_idx, key_idx):
    if q.dim() != 3 or q_idx.dim() != 2 or key_idx.dim() != 2:
        raise ValueError("q/k/v must be [T, H, D], q_idx [Ct, cs], key_idx [Ct, nk]")
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    T, H, D = q.shape
    Ct, cs = q_idx.shape
    if key_idx.shape[0] != Ct:
        raise ValueError("q_idx and key_idx must have one row per cluster")
    return T, H, D, Ct, cs, key_idx.shape[1]


def fwd_varlen(q, k, v, q_idx, key_idx, scale: float | None = None):
    """Forward of a packed batch: O [T, H, D] (dtype of q), LSE [T, H] f32."""
    lib = _lib.load()
    T, H, D, Ct, cs, nk = _varlen_shapes(q, q_idx, key_idx)
    for t, n in ((k, "k"), (v, "v")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q in shape and dtype")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _check(lib.cluster_attn_fwd_varlen(
        _DT[q.dtype], T, Ct, H, D, cs, nk, scale, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
        _dev(q_idx, "q_idx", torch.int32), _dev(key_idx, "key_idx", torch.int32),
        o.data_ptr(), lse.data_ptr(), _stream(q)), "cluster_attn_fwd_varlen")
    return o, lse


def bwd_varlen(q, k, v, o, do, lse, q_idx, key_idx, scale: float | None = None,
               workspace: torch.Tensor | None = None, plan: torch.Tensor | None = None):
    """Backward of a packed batch: dQ, dK, dV [T, H, D] (dtype of q);
    ``plan`` as for :func:`bwd` (from ``bwd_plan(q_idx, key_idx, T)``)."""
    lib = _lib.load()
    T, H, D, Ct, cs, nk = _varlen_shapes(q, q_idx, key_idx)
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (do, "do")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q in shape and dtype")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dt = _DT[q.dtype]
    if plan is not None:
        return _bwd_planned(lib, dt, 1, T, Ct, H, D, cs, nk, scale, q, k, v, o, do, lse, q_idx,
                            key_idx, plan, workspace)
    need = lib.cluster_attn_bwd_varlen_workspace(dt, T, Ct, H, D, cs, nk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _check(lib.cluster_attn_bwd_varlen(
        dt, T, Ct, H, D, cs, nk, scale, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"),
        _dev(do, "do"), _dev(lse, "lse", torch.float32), _dev(q_idx, "q_idx", torch.int32),
        _dev(key_idx, "key_idx", torch.int32), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(q)), "cluster_attn_bwd_varlen")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# KNN-cache point sampler (decoder)
# ---------------------------------------------------------------------------

def knn_table_workspace_bytes(B: int, N: int, grid_side: int) -> int:
    return int(_lib.load().cluster_attn_knn_table_workspace(B, N, grid_side))


def knn_table(coords: torch.Tensor, grid_side: int, K: int,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """[B, G, G, K] int32 table of the K nearest tokens of every grid cell.

    coords: [B, N, 2] float32 device tensor (x = column, y = row).  Images
    above 4096 tokens need a workspace (allocated here when not given)."""
    lib = _lib.load()
    if coords.dim() != 3 or coords.shape[2] != 2:
        raise ValueError("coords must be [B, N, 2]")
    B, N, _ = coords.shape
    G = int(grid_side)
    need = lib.cluster_attn_knn_table_workspace(B, N, G)
    ws_ptr, ws_n = 0, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=coords.device)
        ws_ptr, ws_n = workspace.data_ptr(), workspace.numel()
    table = torch.empty((B, G, G, K), dtype=torch.int32, device=coords.device)
    _check(lib.cluster_attn_knn_table(_dev(coords, "coords", torch.float32), B, N, G, K,
                                      table.data_ptr(), ws_ptr, ws_n, _stream(coords)),
           "cluster_attn_knn_table")
    return table


def _knn_shapes(feats, coords, queries, table):
    if feats.dim() != 3 or coords.dim() != 3 or queries.dim() != 3 or table.dim() != 4:
        raise ValueError("feats [B, N, C], coords [B, N, 2], queries [B, M, 2], table [B, G, G, K]")
    B, N, C = feats.shape
    M = queries.shape[1]
    G, K = table.shape[1], table.shape[3]
    if coords.shape != (B, N, 2) or queries.shape != (B, M, 2) or table.shape != (B, G, G, K):
        raise ValueError("inconsistent shapes")
    if feats.dtype not in _DT:
        raise TypeError(f"unsupported dtype {feats.dtype}")
    return B, N, M, C, G, K


def knn_sample_fwd(feats, coords, queries, table, p: float) -> torch.Tensor:
    """out [B, M, C] (dtype of feats) = softmax(-p d)-weighted sum of the
    table slots of every query's nearest cell."""
    lib = _lib.load()
    B, N, M, C, G, K = _knn_shapes(feats, coords, queries, table)
    out = torch.empty((B, M, C), dtype=feats.dtype, device=feats.device)
    _check(lib.cluster_attn_knn_sample_fwd(
        _DT[feats.dtype], B, N, M, C, G, K, float(p), _dev(coords, "coords", torch.float32),
        _dev(feats, "feats"), _dev(queries, "queries", torch.float32),
        _dev(table, "table", torch.int32), out.data_ptr(), _stream(feats)),
        "cluster_attn_knn_sample_fwd")
    return out


def knn_bwd_workspace_bytes(B: int, N: int, M: int, K: int) -> int:
    return int(_lib.load().cluster_attn_knn_sample_bwd_workspace(B, N, M, K))


def knn_sample_bwd(feats, coords, queries, table, p: float, dout,
                   workspace: torch.Tensor | None = None):
    """Returns dfeats [B, N, C] (dtype of feats), dq [B, M, 2] f32 and dp
    (a one-element f32 device tensor)."""
    lib = _lib.load()
    B, N, M, C, G, K = _knn_shapes(feats, coords, queries, table)
    if dout.shape != (B, M, C) or dout.dtype != feats.dtype:
        raise ValueError("dout must be [B, M, C] in the dtype of feats")
    need = lib.cluster_attn_knn_sample_bwd_workspace(B, N, M, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=feats.device)
    dfeats = torch.empty_like(feats)
    dq = torch.empty((B, M, 2), dtype=torch.float32, device=feats.device)
    dp = torch.empty((1,), dtype=torch.float32, device=feats.device)
    _check(lib.cluster_attn_knn_sample_bwd(
        _DT[feats.dtype], B, N, M, C, G, K, float(p), _dev(coords, "coords", torch.float32),
        _dev(feats, "feats"), _dev(queries, "queries", torch.float32),
        _dev(table, "table", torch.int32), _dev(dout, "dout"), dfeats.data_ptr(), dq.data_ptr(),
        dp.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(feats)),
        "cluster_attn_knn_sample_bwd")
    return dfeats, dq, dp


class _KnnSample(torch.autograd.Function):
    @staticmethod
    def forward(ctx, feats, coords, queries, table, p):
        out = knn_sample_fwd(feats, coords, queries, table, p)
        ctx.save_for_backward(feats, coords, queries, table)
        ctx.p = p
        return out

    @staticmethod
    def backward(ctx, dout):
        feats, coords, queries, table = ctx.saved_tensors
        dfeats, dq, _ = knn_sample_bwd(feats, coords, queries, table, ctx.p, dout.contiguous())
        return dfeats, None, dq, None, None


def knn_sample(feats, coords, queries, table, p: float):
    """Autograd-aware sampler (gradients for feats and queries; the table
    and the token coordinates are constants)."""
    return _KnnSample.apply(feats, coords, queries, table, p)


# ---------------------------------------------------------------------------
# Adaptive token merging
# ---------------------------------------------------------------------------

def merge_plan_workspace_bytes(B: int, N: int, k: int) -> int:
    return int(_lib.load().cluster_attn_merge_plan_workspace(B, N, k))


def merge_plan(coords: torch.Tensor, scores: torch.Tensor, k: int, grid_side: int,
               workspace: torch.Tensor | None = None):
    """Anchors [B, k], assignment [B, N], member lists [B, N] and group
    offsets [B, k + 1] (all int32).  Images above 4096 tokens need a
    workspace (allocated here when not given)."""
    lib = _lib.load()
    if coords.dim() != 3 or coords.shape[2] != 2 or scores.shape != coords.shape[:2]:
        raise ValueError("coords [B, N, 2] and scores [B, N] expected")
    B, N, _ = coords.shape
    dev = coords.device
    need = lib.cluster_attn_merge_plan_workspace(B, N, int(k))
    ws_ptr, ws_n = 0, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr, ws_n = workspace.data_ptr(), workspace.numel()
    anchors = torch.empty((B, k), dtype=torch.int32, device=dev)
    assign = torch.empty((B, N), dtype=torch.int32, device=dev)
    members = torch.empty((B, N), dtype=torch.int32, device=dev)
    offsets = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    _check(lib.cluster_attn_merge_plan(
        _dev(coords, "coords", torch.float32), _dev(scores, "scores", torch.float32), B, N, int(k),
        int(grid_side), anchors.data_ptr(), assign.data_ptr(), members.data_ptr(),
        offsets.data_ptr(), ws_ptr, ws_n, _stream(coords)), "cluster_attn_merge_plan")
    return anchors, assign, members, offsets


def merge_fwd(feats, coords, scores, members, offsets):
    """Merged features [B, k, C] (dtype of feats) and coordinates [B, k, 2] f32."""
    lib = _lib.load()
    B, N, C = feats.shape
    k = offsets.shape[1] - 1
    if feats.dtype not in _DT:
        raise TypeError(f"unsupported dtype {feats.dtype}")
    out_f = torch.empty((B, k, C), dtype=feats.dtype, device=feats.device)
    out_x = torch.empty((B, k, 2), dtype=torch.float32, device=feats.device)
    _check(lib.cluster_attn_merge_fwd(
        _DT[feats.dtype], B, N, k, C, _dev(feats, "feats"), _dev(coords, "coords", torch.float32),
        _dev(scores, "scores", torch.float32), _dev(members, "members", torch.int32),
        _dev(offsets, "offsets", torch.int32), out_f.data_ptr(), out_x.data_ptr(),
        _stream(feats)), "cluster_attn_merge_fwd")
    return out_f, out_x


def merge_bwd(feats, coords, scores, members, offsets, dout_feats, dout_coords):
    """Gradients of features (dtype of feats), coordinates and scores (f32)."""
    lib = _lib.load()
    B, N, C = feats.shape
    k = offsets.shape[1] - 1
    if dout_feats.shape != (B, k, C) or dout_feats.dtype != feats.dtype:
        raise ValueError("dout_feats must be [B, k, C] in the dtype of feats")
    dfeats = torch.empty_like(feats)
    dcoords = torch.empty((B, N, 2), dtype=torch.float32, device=feats.device)
    dscores = torch.empty((B, N), dtype=torch.float32, device=feats.device)
    _check(lib.cluster_attn_merge_bwd(
        _DT[feats.dtype], B, N, k, C, _dev(feats, "feats"), _dev(coords, "coords", torch.float32),
        _dev(scores, "scores", torch.float32), _dev(members, "members", torch.int32),
        _dev(offsets, "offsets", torch.int32), _dev(dout_feats, "dout_feats"),
        _dev(dout_coords, "dout_coords", torch.float32), dfeats.data_ptr(), dcoords.data_ptr(),
        dscores.data_ptr(), _stream(feats)), "cluster_attn_merge_bwd")
    return dfeats, dcoords, dscores
