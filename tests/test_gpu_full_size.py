"""Full-size GPU parity: the Llama-3.1-8B, Qwen3-14B/32B and Llama-3.3-70B layer shapes,
in the launch configurations bench.py times, compared with the oracle on EVERY row.

* Single projections: weights generated on the device and packed by the GPU; column
  norms, masks and values bit-exact against the oracle's pack of the same weights, the
  SpMV and the dense GEMV within |y - y_ref| <= 1e-2 |y_ref| + 1e-3 sum_j |W_ij x_j|
  on all R outputs.
* The fused launches of the decode step: q|k|v through nm_spmv_multi and gate|up
  through nm_spmv_swiglu at the 8B and 70B shapes, every output.
* Launch-plan coverage: every distinct launch plan (kernel, workgroup size, row
  splits, tiles per step, epilogue, batch size) among the launches bench.py times is
  run once at its own shape and checked against the oracle on all rows, so a planner
  change cannot leave a timed kernel instance without a parity test.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_as_f64, host_bf16, host_f32, host_u32, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402

RTOL, ATOL_FRAC = 1e-2, 1e-3
THREADS = 16  # the oracle's row split over host threads (each output is still one sequential sum)


def assert_within(y_bits, y_ref, absum, what):
    y = bf16_as_f64(y_bits)
    ok = oracle.within_tolerance(y, y_ref, absum, RTOL, ATOL_FRAC)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance, e.g. {i}: "
                             f"gpu={y[i]!r} ref={y_ref[i]!r}")


def assert_h(h_bits, g, ag, u, au, what):
    h = bf16_as_f64(h_bits)
    ref = oracle.swiglu(g, u)
    ok = np.abs(h - ref) <= oracle.swiglu_tolerance(g, ag, u, au)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside, e.g. {i}: gpu={h[i]} ref={ref[i]}")


_pack_cache: dict = {}


def device_layer(R, K, N, M, *ids):
    """Device weights, calibration norms and the GPU pack of one layer, plus the oracle's
    pack of the same weights (cached for the last layer: the B = 1 and B = 4 cases of one
    shape share it)."""
    key = (R, K, N, M, ids)
    Wd = synth.device_weights(R, K, 0, R, K, *ids)
    Xd = synth.device_calib_acts(K, 0, K, *ids)
    n = nm.nm_col_norm(Xd)
    masks, values = nm.nm_prune_pack(Wd, n, N, M)
    torch.cuda.synchronize()
    if key not in _pack_cache:
        _pack_cache.clear()
        W = host_bf16(Wd)
        nref = oracle.col_norm(host_bf16(Xd))
        mref, vref = oracle.prune_pack(W, nref, N, M)
        _pack_cache[key] = (W, nref, mref, vref)
    W, nref, mref, vref = _pack_cache[key]
    assert (host_f32(n).view(np.uint32) == nref.view(np.uint32)).all(), "column norms"
    assert (host_u32(masks) == mref).all(), "masks"
    assert (host_bf16(values) == vref).all(), "values"
    return Wd, (masks, values), W, (mref, vref)


# (name, R, K, N, M, B): the single-projection launches of the bench's layer sets
FULL = [
    ("8b-q", 4096, 4096, 2, 4, 1), ("8b-kv", 1024, 4096, 16, 32, 1), ("8b-up", 14336, 4096, 2, 4, 1),
    ("8b-down", 4096, 14336, 16, 32, 1), ("8b-gate-b8", 14336, 4096, 2, 4, 8),
    ("14b-up", 17408, 5120, 4, 8, 1), ("14b-down", 5120, 17408, 4, 8, 1),
    ("32b-q", 8192, 5120, 4, 8, 1), ("32b-down", 5120, 25600, 4, 8, 1),
    ("70b-kv", 1024, 8192, 8, 16, 8), ("70b-q-b2", 8192, 8192, 8, 16, 2),
    ("70b-down", 8192, 28672, 8, 16, 1), ("70b-down-b4", 8192, 28672, 8, 16, 4),
    ("70b-up-b8", 28672, 8192, 8, 16, 8),
]


@pytest.mark.parametrize("name,R,K,N,M,B", FULL, ids=[f[0] for f in FULL])
def test_full_size_all_rows(name, R, K, N, M, B):
    say("full", name, R, K, N, M, B, nm.nm_spmv_plan(R, K, B))
    Wd, (masks, values), W, (mref, vref) = device_layer(R, K, N, M)
    xd = synth.device_decode_x(B, K, 0, K, B)
    y = nm.nm_spmv(masks, values, xd)
    yd = nm.dense_gemv(Wd, xd)
    torch.cuda.synchronize()
    xh = host_bf16(xd)
    yref, absum = oracle.spmv(mref, vref, xh, K, nthreads=THREADS)
    assert_within(host_bf16(y), yref, absum, f"{name} sparse")
    ydref, adabs = oracle.dense(W, xh, nthreads=THREADS)
    assert_within(host_bf16(yd), ydref, adabs, f"{name} dense")


# ------------------------------------------------------------------ the step's fused launches
@pytest.mark.parametrize("K,Rs,B", [(4096, (4096, 1024, 1024), 1), (4096, (4096, 1024, 1024), 8),
                                    (8192, (8192, 1024, 1024), 1), (8192, (8192, 1024, 1024), 8)],
                         ids=["8b-b1", "8b-b8", "70b-b1", "70b-b8"])
def test_qkv_launch_all_rows(K, Rs, B):
    """q|k|v of one decoder layer in one nm_spmv_multi launch, as the decode step runs it."""
    say("qkv launch", K, Rs, B, nm.nm_spmv_multi_plan(Rs, K, B))
    N, M = (2, 4) if K == 4096 else (8, 16)
    layers = [device_layer(R, K, N, M, 40 + i) for i, R in enumerate(Rs)]
    xd = synth.device_decode_x(B, K, 0, 41, B)
    ys = nm.nm_spmv_multi([lay[1] for lay in layers], xd)
    dys = nm.dense_gemv_multi([lay[0] for lay in layers], xd)
    torch.cuda.synchronize()
    xh = host_bf16(xd)
    for i, (lay, y, dy) in enumerate(zip(layers, ys, dys)):
        yref, absum = oracle.spmv(*lay[3], xh, K, nthreads=THREADS)
        assert_within(host_bf16(y), yref, absum, f"qkv matrix {i}")
        dref, dabs = oracle.dense(lay[2], xh, nthreads=THREADS)
        assert_within(host_bf16(dy), dref, dabs, f"dense qkv matrix {i}")


@pytest.mark.parametrize("R,K,B", [(14336, 4096, 1), (14336, 4096, 8), (28672, 8192, 1)],
                         ids=["8b-b1", "8b-b8", "70b-b1"])
def test_gate_up_launch_all_rows(R, K, B):
    """gate|up with the SiLU-and-multiply epilogue in one nm_spmv_swiglu launch."""
    say("gate|up launch", R, K, B, nm.nm_spmv_plan(R, K, B, nm.NM_EPI_SWIGLU))
    N, M = (2, 4) if K == 4096 else (8, 16)
    Wg, gate, Wgh, gref = device_layer(R, K, N, M, 50)
    g_all = gref  # keep the oracle pack of gate before the cache moves on to up
    Wu, up, Wuh, uref = device_layer(R, K, N, M, 51)
    xd = synth.device_decode_x(B, K, 0, 52, B)
    h = nm.nm_spmv_swiglu(gate, up, xd)
    hd = nm.dense_gemv_swiglu(Wg, Wu, xd)
    torch.cuda.synchronize()
    xh = host_bf16(xd)
    g, ag = oracle.spmv(*g_all, xh, K, nthreads=THREADS)
    u, au = oracle.spmv(*uref, xh, K, nthreads=THREADS)
    assert_h(host_bf16(h), g, ag, u, au, "sparse gate|up")
    g, ag = oracle.dense(Wgh, xh, nthreads=THREADS)
    u, au = oracle.dense(Wuh, xh, nthreads=THREADS)
    assert_h(host_bf16(hd), g, ag, u, au, "dense gate|up")


# ------------------------------------------------------------------ launch-plan coverage
def bench_launches():
    """(kind, rows, K, B) of every launch bench.py times: single projections, q|k|v
    (rows of each matrix) and gate|up (rows of each), for every layer set and batch size
    its configurations name."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import bench

    out = set()
    for cname, cfg in bench.CONFIGS.items():
        projs = cfg.get("projs") or bench.CONFIGS[cfg["base"]]["projs"]
        for B in cfg["batch"]:
            for name, R, K, _ in projs:
                out.add(("one", (R,), K, B))
            groups = {}
            for name, R, K, grp in projs:
                groups.setdefault(grp, []).append((name, R, K))
            for grp in groups.values():
                names = [g[0] for g in grp]
                if names == ["gate", "up"]:
                    out.add(("swiglu", (grp[0][1],), grp[0][2], B))
                elif len(grp) > 1:
                    out.add(("multi", tuple(g[1] for g in grp), grp[0][2], B))
    return sorted(out)


def plan_signature(kind, rows, K, B):
    if kind == "multi":
        p = nm.nm_spmv_multi_plan(list(rows), K, B)
    else:
        p = nm.nm_spmv_plan(rows[0], K, B, nm.NM_EPI_SWIGLU if kind == "swiglu" else nm.NM_EPI_NONE)
    return (kind, B, p["kernel"], p["threads"], p["splits"] > 1, p["tiles_per_step"], p["x_steps_in_registers"])


def coverage_cases():
    rep = {}
    for kind, rows, K, B in bench_launches():
        sig = plan_signature(kind, rows, K, B)
        size = sum(rows) * K
        if sig not in rep or size < rep[sig][0]:
            rep[sig] = (size, kind, rows, K, B)
    return [(sig, v[1:]) for sig, v in sorted(rep.items())]


def test_bench_launch_classes_listed():
    cases = coverage_cases()
    say("launch classes", len(cases))
    assert len(cases) >= 8
    kinds = {sig[0] for sig, _ in cases}
    assert kinds == {"one", "multi", "swiglu"}


CLASSES = coverage_cases()  # the planner runs on the host: known at collection time


@pytest.mark.parametrize("sig,case", CLASSES,
                         ids=[f"{s[0]}-B{s[1]}-k{s[2]}-t{s[3]}{'-split' if s[4] else ''}-tt{s[5]}-x{s[6]}"
                              for s, _ in CLASSES])
def test_bench_launch_class_parity(sig, case):
    """One launch of each distinct plan the bench times, at its own shape, all rows: the
    product against the oracle's matvec of the GPU-packed operands (the pack itself is
    held bit-exact by the tests above)."""
    kind, rows, K, B = case
    say("launch class", sig, kind, rows, K, B)
    n = nm.nm_col_norm(synth.device_calib_acts(K, 0, 60, K))
    mats = []
    for i, R in enumerate(rows if kind != "swiglu" else (rows[0], rows[0])):
        W = synth.device_weights(R, K, 0, 61, i, R, K)
        mats.append(nm.nm_prune_pack(W, n, 4, 8))
        del W
    xd = synth.device_decode_x(B, K, 0, 62, B)
    if kind == "one":
        outs = [nm.nm_spmv(*mats[0], xd)]
    elif kind == "multi":
        outs = nm.nm_spmv_multi(mats, xd)
    else:
        outs = [nm.nm_spmv_swiglu(mats[0], mats[1], xd)]
    torch.cuda.synchronize()
    xh = host_bf16(xd)
    refs = [oracle.spmv(host_u32(m), host_bf16(v), xh, K, nthreads=THREADS) for m, v in mats]
    if kind == "swiglu":
        assert_h(host_bf16(outs[0]), *refs[0], *refs[1], f"class {sig}")
    else:
        for i, (y, (yref, absum)) in enumerate(zip(outs, refs)):
            assert_within(host_bf16(y), yref, absum, f"class {sig} matrix {i}")


@pytest.mark.parametrize("B", [1, 2, 8])
def test_values_beyond_2gib(B):
    """A matrix whose packed values pass 2^31 bytes (270000 x 8192: 2.2 GB of values, 4.4 GB
    of dense weights), so row offsets need more than 32 bits in the pack and in every walk
    (B = 1: strips of consecutive rows per workgroup; B = 2: whole rows per wave; B = 8:
    matrix cores, 16875 tiles, several units per workgroup): masks and values bit-exact and
    outputs within tolerance on sampled rows, the first and last rows included."""
    R, K = 270000, 8192
    say("beyond 2 GiB", R, K, B)
    plan = nm.nm_spmv_plan(R, K, B)
    assert plan["kernel"] == {1: nm.NM_KERNEL_WORD_STRIPS, 2: nm.NM_KERNEL_WORD, 8: nm.NM_KERNEL_TILE}[B]
    Wd = synth.device_weights(R, K, 0, 61, R, K)
    Xd = synth.device_calib_acts(K, 0, 61, K)
    n = nm.nm_col_norm(Xd)
    masks, values = nm.nm_prune_pack(Wd, n, 8, 16)
    assert values.numel() * 2 > 2 ** 31
    xd = synth.device_decode_x(B, K, 0, 61, B)
    y = nm.nm_spmv(masks, values, xd)
    torch.cuda.synchronize()
    g = np.random.default_rng(61)
    rows = np.unique(np.concatenate([[0, 1, R // 2, R - 2, R - 1], g.choice(R, size=250, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    W = host_bf16(Wd.index_select(0, ridx))
    del Wd
    nref = oracle.col_norm(host_bf16(Xd))
    assert (host_f32(n).view(np.uint32) == nref.view(np.uint32)).all(), "column norms"
    mref, vref = oracle.prune_pack(W, nref, 8, 16)
    assert (host_u32(masks.index_select(0, ridx)) == mref).all(), "masks"
    assert (host_bf16(values.index_select(0, ridx)) == vref).all(), "values"
    yref, absum = oracle.spmv(mref, vref, host_bf16(xd), K, nthreads=THREADS)
    assert_within(host_bf16(y)[:, rows], yref, absum, f"{R}x{K} B={B}")
