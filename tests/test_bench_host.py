"""Host-side logic of bench.py (no GPU): the algorithmic byte counts the
roofline divides by, the rotation sizing and the per-launch timing choice."""

import bench
from gen import CONFIGS


def test_algorithmic_bytes_match_the_scope_table():
    # stage-1: 65,536 tokens x 4 heads; forward 267 B and backward 523 B per
    # (query, head), i.e. 69,992,448 and 137,101,312 bytes per launch
    alg = bench.algorithmic(CONFIGS["stage1"])
    assert alg["fwd"]["bytes"] == 69_992_448
    assert alg["bwd"]["bytes"] == 137_101_312
    # QK^T + PV on 48 slots of 32 dims, and five such products backward
    assert alg["fwd"]["flops"] == 65536 * 4 * 4 * 48 * 32
    assert alg["bwd"]["flops"] == 65536 * 4 * 10 * 48 * 32


def test_rotation_walks_twice_the_last_level_cache():
    cfg = CONFIGS["stage1"]
    tensor = cfg.B * cfg.N * cfg.H * cfg.D * 2
    n = bench.rotation_copies(0, tensor)
    assert n * 3 * tensor >= 2 * (256 << 20)
    assert bench.rotation_copies(7, tensor) == 7


def _st(m):
    return {"mean": m, "median": m, "p10": m, "p90": m}


def test_pick_timing_takes_the_faster_launch_mode():
    graph = {"a": _st(10.0), "b": _st(5.0), "c": None}
    stream = {"a": _st(9.0), "b": _st(6.0), "c": _st(7.0)}
    stats, how = bench.pick_timing(["a", "b", "c"], graph, stream)
    assert stats["a"]["mean"] == 9.0 and how["a"].startswith("stream")
    assert stats["b"]["mean"] == 5.0 and how["b"].startswith("graph")
    assert stats["c"]["mean"] == 7.0 and how["c"].startswith("stream")
    stats, how = bench.pick_timing(["a"], None, stream)
    assert stats["a"]["mean"] == 9.0 and how["a"].startswith("stream")


def test_formulation_bytes_drop_the_unread_output():
    cfg = CONFIGS["stage1"]
    alg = bench.algorithmic(cfg)
    f = bench.formulation_bytes(cfg, "bwd", alg, {"bwd": 50.0})
    assert f["bytes_this_formulation_moves"] == 137_101_312 - 65536 * 4 * 32 * 2
    assert bench.formulation_bytes(cfg, "fwd", alg, {"fwd": 20.0}) == {}
