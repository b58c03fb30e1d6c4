"""Every output element at the launch configuration the benchmark times.

The benchmark runs whole batches (stage-1, stage-2, stage-3, stage-4, the
stress workload and the 3D volumes at B = 32, high-res at B = 4) through
the forward and the planned backward,
where every wavefront walks several items.  These tests run exactly those
launches and compare every element of O, LSE, dQ, dK and dV with the fp64
oracle (gathered form, cluster blocks); high-res compares one whole image.
They also run a batch size that leaves an uneven number of items per
wavefront, check that a second forward / backward on the same inputs is
bitwise identical, and assert two sum rules that hold at any size.

Bars.  bf16 workloads: the stated tolerances (O 1e-2, gradients 2e-2 abs,
LSE 1e-3).  The fp16 x8 stress workload: the scale-relative reading (O
1e-2 * max(1, max|O|), gradients 2e-2 * max(1, max|g|), LSE 1e-2), and in
addition an element-wise bar from fp16 arithmetic, u = 2^-11 being the unit
roundoff of fp16: each output is a rounded sum of products, whose error is
bounded by u times the sum of the term magnitudes (parity_util's
term_magnitudes, which folds in the error of Delta from the rounded O).
Per term: the rounding of its probability or dS operand (u, or at most
2^-25 absolute where the operand falls below fp16's normal range) and the
fp32 logits at |logit| <= ~350 (32-term dot products: well under u relative
on a probability); per element: one output rounding (u |ref|).  So
  |err| <= 2u |ref| + 2u * sum|terms| + 2^-24 * sum|other operand|.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from gen import make_case, make_volume_case, stress_duplicate_slots
from gen.synth import stress_rng
from parity_util import assert_finite, check_close, term_magnitudes, to_np, tol_for

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U16 = 2.0 ** -11


@pytest.fixture(scope="module")
def ca():
    import gathered_local_attention_amd as ca

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ca._lib.load()
    return ca


def _lists(ca, case, images=None):
    """GPU lists for the whole batch; oracle lists for ``images`` (all by
    default), which must be identical to the GPU's."""
    cfg = case["cfg"]
    perm, _, key = ca.build_neighbors(torch.from_numpy(case["coords"]).to(DEV), cfg.G)
    torch.cuda.synchronize()
    sel = slice(None) if images is None else images
    perm_r, _, key_r = O.build_neighbors(case["coords"][sel], cfg.G)
    assert np.array_equal(perm.cpu().numpy()[sel], perm_r), "perm differs from the oracle"
    assert np.array_equal(key.cpu().numpy()[sel], key_r), "key_idx differs from the oracle"
    key_np = key.cpu().numpy()
    if cfg.dup_frac:
        key_np = stress_duplicate_slots(key_np, cfg.cs, stress_rng(cfg), cfg.dup_frac)
        key = torch.from_numpy(key_np).to(DEV)
    return perm, key, perm.cpu().numpy().reshape(cfg.B, cfg.C, cfg.cs), key_np


def _run(ca, case, perm, key):
    """The benchmark's launches: forward, then the backward on a plan built
    once from the lists."""
    cfg = case["cfg"]
    scale = 1.0 / math.sqrt(cfg.D)
    q, k, v, do = (case[n].to(DEV) for n in ("q", "k", "v", "do"))
    plan = ca.bwd_plan(perm, key, cfg.N)
    o, lse = ca.fwd(q, k, v, perm, key, scale)
    dq, dk, dv = ca.bwd(q, k, v, o, do, lse, perm, key, scale, plan=plan)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, q=q, k=k, v=v, do=do, plan=plan, scale=scale)


def _elementwise_fp16(name, got, ref, mag, floor):
    """The derived fp16 element-wise bar (see the module docstring)."""
    g = to_np(got)
    bar = 2 * U16 * np.abs(ref) + 2 * U16 * mag + 2.0 ** -24 * floor + 1e-30
    ratio = float((np.abs(g - ref) / bar).max())
    print(f"  {name}: worst err / element-wise fp16 bar = {ratio:.3f}", flush=True)
    assert ratio <= 1.0, f"{name}: element-wise error above the fp16 bar (ratio {ratio:.3f})"


def _compare(cfg, r, ref_o, ref_lse, ref_g, sel=slice(None), mag=None):
    tol = tol_for(cfg)
    for nm in ("o", "lse", "dq", "dk", "dv"):
        assert_finite(nm, r[nm])
    check_close("O", r["o"][sel], ref_o, tol["o"], tol["rel"])
    check_close("LSE", r["lse"][sel], ref_lse, tol["lse"], False)
    for nm, key, ref in zip(("dQ", "dK", "dV"), ("dq", "dk", "dv"), ref_g):
        check_close(nm, r[key][sel], ref, tol["g"], tol["rel"])
    if mag is not None:
        _elementwise_fp16("O", r["o"][sel], ref_o, mag["o"], mag["o_floor"])
        for nm, key, ref in zip(("dQ", "dK", "dV"), ("dq", "dk", "dv"), ref_g):
            _elementwise_fp16(nm, r[key][sel], ref, mag[key], mag[key + "_floor"])


def _sum_rules(cfg, r):
    """Sum over the tokens of an image: dK sums to 0 (a shift of every key
    moves no probability) and dV sums to the sum of dO (each probability row
    sums to 1), per image, head and dim.  Output rounding puts at most
    2^-9 |x| (bf16; 2^-11 fp16) on each element and the rounded P/dS
    operands at most as much again, so the sums may be off by at most twice
    that over the magnitudes summed."""
    u = 2.0 ** -9 if cfg.dtype == "bf16" else 2.0 ** -11
    dk, dv, do = (r[n].double() for n in ("dk", "dv", "do"))
    s_dk = dk.sum(dim=1).abs()
    b_dk = 2 * u * dk.abs().sum(dim=1) + 1e-6
    s_dv = (dv.sum(dim=1) - do.sum(dim=1)).abs()
    b_dv = 2 * u * (dv.abs().sum(dim=1) + do.abs().sum(dim=1)) + 1e-6
    rk, rv = float((s_dk / b_dk).max()), float((s_dv / b_dv).max())
    print(f"  sum rules: |sum dK| / bound {rk:.3f}, |sum dV - sum dO| / bound {rv:.3f}",
          flush=True)
    assert rk <= 1.0 and rv <= 1.0


@pytest.mark.parametrize("name,B", [("stage1", 32), ("stage3", 32), ("stress", 32), ("stage1", 19),
                                    ("stage2", 32), ("stage4", 32)])
def test_whole_batch_every_element(ca, name, B):
    case = make_case(name, B=B)
    cfg = case["cfg"]
    print(f"case {name} B={cfg.B} N={cfg.N} H={cfg.H} {cfg.dtype} (every element)", flush=True)
    perm, key, qi, key_np = _lists(ca, case)
    r = _run(ca, case, perm, key)
    ref_o, ref_lse = O.attn_fwd_gathered(case["q"], case["k"], case["v"], qi, key_np, r["scale"])
    ref_g = O.attn_bwd_gathered(case["q"], case["k"], case["v"], case["do"], qi, key_np,
                                r["scale"])
    mag = None
    if cfg.qkv_scale != 1.0:
        mag = term_magnitudes(case["q"], case["k"], case["v"], case["do"], qi, key_np, r["scale"])
    _compare(cfg, r, ref_o, ref_lse, ref_g, mag=mag)
    _sum_rules(cfg, r)


def test_volume_whole_batch_every_element(ca):
    """The 32-volume 3D batch as the benchmark runs it (lists from the 3D
    build, bit-exact), every element against the oracle."""
    case = make_volume_case("volume")
    cfg = case["cfg"]
    print(f"case volume B={cfg.B} N={cfg.N} (3D, every element)", flush=True)
    perm, _, key = ca.build_neighbors(torch.from_numpy(case["coords"]).to(DEV), cfg.G)
    torch.cuda.synchronize()
    perm_r, _, key_r = O.build_neighbors_3d(case["coords"], cfg.G)
    assert np.array_equal(perm.cpu().numpy(), perm_r), "perm differs from the oracle"
    assert np.array_equal(key.cpu().numpy(), key_r), "key_idx differs from the oracle"
    r = _run(ca, case, perm, key)
    qi = perm_r.reshape(cfg.B, -1, cfg.cs)
    ref_o, ref_lse = O.attn_fwd_gathered(case["q"], case["k"], case["v"], qi, key_r, r["scale"])
    ref_g = O.attn_bwd_gathered(case["q"], case["k"], case["v"], case["do"], qi, key_r,
                                r["scale"])
    _compare(cfg, r, ref_o, ref_lse, ref_g)
    _sum_rules(cfg, r)


def test_volume_hr_whole_volume_every_element(ca):
    """The two 64,000-token volumes as the benchmark runs them; volume 0 is
    compared element by element (lists of both bit-exact)."""
    case = make_volume_case("volume_hr")
    cfg = case["cfg"]
    print(f"case volume_hr B={cfg.B} N={cfg.N} (3D, volume 0, every element)", flush=True)
    perm, _, key = ca.build_neighbors(torch.from_numpy(case["coords"]).to(DEV), cfg.G)
    torch.cuda.synchronize()
    perm_r, _, key_r = O.build_neighbors_3d(case["coords"], cfg.G)
    assert np.array_equal(perm.cpu().numpy(), perm_r), "perm differs from the oracle"
    assert np.array_equal(key.cpu().numpy(), key_r), "key_idx differs from the oracle"
    r = _run(ca, case, perm, key)
    qi = perm_r.reshape(cfg.B, -1, cfg.cs)
    one = lambda t: t[0:1]
    ref_o, ref_lse = O.attn_fwd_gathered(one(case["q"]), one(case["k"]), one(case["v"]),
                                         qi[0:1], key_r[0:1], r["scale"])
    ref_g = O.attn_bwd_gathered(one(case["q"]), one(case["k"]), one(case["v"]), one(case["do"]),
                                qi[0:1], key_r[0:1], r["scale"])
    _compare(cfg, r, ref_o, ref_lse, ref_g, sel=slice(0, 1))
    _sum_rules(cfg, r)


def test_highres_whole_image_every_element(ca):
    """B = 4 images of 65,536 tokens run as the benchmark runs them; image 0
    is compared element by element (the oracle works through it in blocks
    of 1024 clusters)."""
    case = make_case("highres")
    cfg = case["cfg"]
    print(f"case highres B={cfg.B} N={cfg.N} (image 0, every element)", flush=True)
    perm, key, qi, key_np = _lists(ca, case, images=slice(0, 1))
    r = _run(ca, case, perm, key)
    one = lambda t: t[0:1]
    ref_o, ref_lse = O.attn_fwd_gathered(one(case["q"]), one(case["k"]), one(case["v"]),
                                         qi[0:1], key_np[0:1], r["scale"])
    ref_g = O.attn_bwd_gathered(one(case["q"]), one(case["k"]), one(case["v"]), one(case["do"]),
                                qi[0:1], key_np[0:1], r["scale"])
    _compare(cfg, r, ref_o, ref_lse, ref_g, sel=slice(0, 1))
    _sum_rules(cfg, r)


@pytest.mark.parametrize("name", ["stage1", "stress"])
def test_whole_batch_bitwise_repeatable(ca, name):
    """Run-to-run bitwise equality at the benchmarked size (no atomics on
    floating-point values anywhere), and the self-planning backward equal
    to the planned one."""
    case = make_case(name)
    cfg = case["cfg"]
    print(f"case {name} B={cfg.B} repeat", flush=True)
    perm, key, _, _ = _lists(ca, case, images=slice(0, 1))
    r = _run(ca, case, perm, key)
    for _ in range(2):
        o, lse = ca.fwd(r["q"], r["k"], r["v"], perm, key, r["scale"])
        g = ca.bwd(r["q"], r["k"], r["v"], r["o"], r["do"], r["lse"], perm, key, r["scale"],
                   plan=r["plan"])
        torch.cuda.synchronize()
        assert torch.equal(o, r["o"]) and torch.equal(lse, r["lse"])
        for a, nm in zip(g, ("dq", "dk", "dv")):
            assert torch.equal(a, r[nm]), f"{nm} differs between runs"
    g = ca.bwd(r["q"], r["k"], r["v"], r["o"], r["do"], r["lse"], perm, key, r["scale"])
    torch.cuda.synchronize()
    for a, nm in zip(g, ("dq", "dk", "dv")):
        assert torch.equal(a, r[nm]), f"self-planning {nm} differs from the planned backward"
