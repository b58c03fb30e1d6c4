"""ctypes loader for libclusterattn.so (argument types only, no logic)."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libclusterattn.so")

_c_int, _c_size, _vp, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

SIGNATURES = {
    "cluster_attn_build_neighbors_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "cluster_attn_build_neighbors": (
        _c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_fwd": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "cluster_attn_bwd_workspace": (
        _c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "cluster_attn_bwd": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_build_neighbors_varlen_workspace": (
        _c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "cluster_attn_build_neighbors_varlen": (
        _c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                 _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_build_neighbors_3d": (
        _c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_build_neighbors_varlen_3d": (
        _c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                 _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_fwd_varlen": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "cluster_attn_bwd_varlen_workspace": (
        _c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "cluster_attn_bwd_varlen": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_bwd_plan_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "cluster_attn_bwd_plan": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_bwd_plan_varlen": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _c_size,
                 _vp]),
    "cluster_attn_bwd_planned_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "cluster_attn_bwd_planned_noalloc_max_rows": (_c_size, []),
    "cluster_attn_bwd_planned_noalloc": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp, _vp, _vp, _vp]),
    "cluster_attn_bwd_planned": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp, _vp, _vp, _vp,
                 _c_size, _vp]),
    "cluster_attn_device_copy": (_c_int, [_vp, _vp, _c_size, _vp]),
    "cluster_attn_check_lists": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "cluster_attn_knn_table_workspace": (_c_size, [_c_int, _c_int, _c_int]),
    "cluster_attn_knn_table": (
        _c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "cluster_attn_knn_sample_fwd": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp]),
    "cluster_attn_knn_sample_bwd_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "cluster_attn_knn_sample_bwd": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _f,
                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_merge_plan_workspace": (_c_size, [_c_int, _c_int, _c_int]),
    "cluster_attn_merge_plan": (
        _c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "cluster_attn_merge_fwd": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "cluster_attn_merge_bwd": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                 _vp, _vp, _vp, _vp]),
    "cluster_attn_status_string": (ctypes.c_char_p, [_c_int]),
    "cluster_attn_last_error": (ctypes.c_char_p, []),
    "cluster_attn_version": (ctypes.c_char_p, []),
}

_LIB = None


class LibraryMissing(RuntimeError):
    pass


def load(path: str | None = None):
    """Load (once) and return the CDLL; raises LibraryMissing if not built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise LibraryMissing(
            f"{p} not found: build it with `python -m gathered_local_attention_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _LIB = lib
    return lib
