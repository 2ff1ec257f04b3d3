"""GPU parity of the matrix-core path of the bitmask SpMV (5 <= B <= 8 tokens, K a
multiple of 1024; at B = 3 or 4 where a row's x is too large for the word-per-lane
kernel's LDS): each 16-row tile of mask words is expanded into a dense tile in LDS by
the fixed 16-step walk and multiplied by the inputs with MFMA.  Held to the same
bars as the word-per-lane path: the oracle's tolerance element by element, exact
equality where the result is an integer or a single weight."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_as_f64, dev_bf16, dev_u32, host_bf16, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402

PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]
RTOL, ATOL_FRAC = 1e-2, 1e-3


def assert_within(y_bits, y_ref, absum, what):
    y = bf16_as_f64(y_bits)
    ok = oracle.within_tolerance(y, y_ref, absum, RTOL, ATOL_FRAC)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside, e.g. {i}: gpu={y[i]} ref={y_ref[i]}")


@pytest.mark.parametrize("N,M", PATTERNS)
@pytest.mark.parametrize("B", [5, 8])
def test_tile_integer_exact(N, M, B):
    """Ternary weights and inputs: every sum is an integer below 2^8, exact in the
    MFMA's bf16 products and fp32 sums and in bf16, so the result equals the oracle's."""
    say("tile integer exact", N, M, B)
    R, K = 300, 1024
    W = synth.ternary((R, K), 30, M, B)
    x = synth.ternary((B, K), 31, M, B)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 30)), N, M)
    y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    yref, _ = oracle.spmv(mref, vref, x, K)
    assert np.abs(yref).max() <= 256
    assert (bf16_as_f64(host_bf16(y)) == yref).all()


def test_tile_one_hot_columns():
    """Token b's input is one-hot at column c_b: y[b] must be column c_b of the pruned
    matrix bit for bit -- each kept value lands at its own column of the dense tile, and
    pruned columns read zero."""
    say("tile one-hot")
    R, K = 999, 4096
    W = synth.weights(R, K, 32)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 32)), 8, 16)
    Wp = oracle.unpack(mref, vref, K)
    cols = [0, 1, 31, 32, 1023, 1029, 2047, 4095]
    x = np.zeros((len(cols), K), np.uint16)
    for b, j in enumerate(cols):
        x[b, j] = 0x3F80  # 1.0
    y = host_bf16(nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x)))
    for b, j in enumerate(cols):
        assert (y[b] == Wp[:, j]).all(), f"column {j}"


@pytest.mark.parametrize("R,K,B", [(1, 1024, 8), (15, 1024, 6), (16, 2048, 7), (17, 3072, 5), (1000, 4096, 8),
                                   (513, 5120, 6), (40, 14336, 8)])
def test_tile_ragged_rows(R, K, B):
    """Row counts that leave the last 16-row tile partly (or mostly) empty."""
    say("tile ragged", R, K, B)
    W = synth.weights(R, K, 33, R, K, B)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 33, R)), 16, 32)
    x = synth.decode_x(B, K, 33, R, K, B)
    y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=4)
    assert_within(host_bf16(y), yref, absum, f"tile R={R} K={K} B={B}")


def test_tile_scaling_and_determinism():
    say("tile scaling + determinism")
    R, K, B = 2048, 4096, 8
    W = synth.weights(R, K, 34)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 34)), 2, 4)
    m, v = dev_u32(mref), dev_bf16(vref)
    x = synth.decode_x(B, K, 34)
    x4 = synth.to_bf16_bits(synth.bf16_bits_to_f32(x) * 4.0)
    y1 = host_bf16(nm.nm_spmv(m, v, dev_bf16(x)))
    y1b = host_bf16(nm.nm_spmv(m, v, dev_bf16(x)))
    y4 = host_bf16(nm.nm_spmv(m, v, dev_bf16(x4)))
    assert (y1 == y1b).all()  # fixed summation order: bit-reproducible
    assert (bf16_as_f64(y4) == 4.0 * bf16_as_f64(y1)).all()
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=4)
    assert_within(y1, yref, absum, "tile 2048x4096")


def test_tile_strided_x_and_y():
    say("tile strided x/y")
    R, K, B = 700, 2048, 7
    W = synth.weights(R, K, 35)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 35)), 4, 8)
    xfull = synth.decode_x(B, K + 64, 35)
    xd = dev_bf16(xfull)[:, :K]
    yfull = torch.zeros((B, R + 40), dtype=torch.bfloat16, device="cuda")
    nm.nm_spmv(dev_u32(mref), dev_bf16(vref), xd, out=yfull[:, :R])
    yh = host_bf16(yfull)
    yref, absum = oracle.spmv(mref, vref, np.ascontiguousarray(xfull[:, :K]), K)
    assert_within(yh[:, :R], yref, absum, "strided")
    assert (yh[:, R:] == 0).all()


@pytest.mark.parametrize("Rs", [[16, 48, 32, 16, 64, 16, 32, 5], [640, 512, 1000], [520, 7, 300]],
                         ids=["aligned8", "aligned3", "unaligned"])
def test_tile_multi_matrix(Rs):
    """Several matrices in one launch: with every matrix but the last a multiple of 16
    rows the set runs on the tile path, otherwise on the word-per-lane path; both give
    each matrix its own oracle result."""
    say("tile multi", Rs)
    K, B = 2048, 8
    x = synth.decode_x(B, K, 36, len(Rs))
    n = oracle.col_norm(synth.calib_acts(K, 36, len(Rs)))
    packed, refs = [], []
    for i, R in enumerate(Rs):
        W = synth.weights(R, K, 36, len(Rs), i)
        mref, vref = oracle.prune_pack(W, n, 8, 16)
        refs.append(oracle.spmv(mref, vref, x, K, nthreads=4))
        packed.append((dev_u32(mref), dev_bf16(vref)))
    ys = nm.nm_spmv_multi(packed, dev_bf16(x))
    for i, (y, (yref, absum)) in enumerate(zip(ys, refs)):
        assert y.shape == (B, Rs[i])
        assert_within(host_bf16(y), yref, absum, f"multi {Rs} matrix {i}")


@pytest.mark.parametrize("R,K,B", [(1, 1024, 8), (9, 1024, 5), (1001, 2048, 6), (128, 4096, 7), (300, 14336, 8)])
def test_tile_swiglu(R, K, B):
    say("tile swiglu", R, K, B)
    n = oracle.col_norm(synth.calib_acts(K, 37, R, K))
    Wg, Wu = synth.weights(R, K, 37, 1, R, K), synth.weights(R, K, 37, 2, R, K)
    gm, gv = oracle.prune_pack(Wg, n, 2, 4)
    um, uv = oracle.prune_pack(Wu, n, 2, 4)
    x = synth.decode_x(B, K, 37, R, K, B)
    h = host_bf16(nm.nm_spmv_swiglu((dev_u32(gm), dev_bf16(gv)), (dev_u32(um), dev_bf16(uv)), dev_bf16(x)))
    g, ag = oracle.spmv(gm, gv, x, K, nthreads=4)
    u, au = oracle.spmv(um, uv, x, K, nthreads=4)
    ref = oracle.swiglu(g, u)
    ok = np.abs(bf16_as_f64(h) - ref) <= oracle.swiglu_tolerance(g, ag, u, au)
    assert ok.all(), f"swiglu R={R} K={K} B={B}: {int((~ok).sum())} outside"


# Launches with enough 16-row tiles (on a 256-CU part: 2048 here) walk two tiles per step
# with one shared x operand; a multi-matrix set does so only when every matrix but the
# last starts at a multiple of 32 rows (else one tile per step).
@pytest.mark.parametrize("Rs", [[32768], [32763], [16384, 16384], [16400, 16368]],
                         ids=["plain", "ragged", "multi32", "multi16"])
def test_tile_two_tiles_per_step(Rs):
    say("tile two per step", Rs)
    K, B = 1024, 8
    x = synth.decode_x(B, K, 38, len(Rs))
    n = oracle.col_norm(synth.calib_acts(K, 38, len(Rs)))
    packed, refs = [], []
    for i, R in enumerate(Rs):
        W = synth.weights(R, K, 38, len(Rs), i)
        mref, vref = oracle.prune_pack(W, n, 4, 8)
        refs.append(oracle.spmv(mref, vref, x, K, nthreads=8))
        packed.append((dev_u32(mref), dev_bf16(vref)))
    ys = nm.nm_spmv_multi(packed, dev_bf16(x)) if len(Rs) > 1 else [nm.nm_spmv(*packed[0], dev_bf16(x))]
    for i, (y, (yref, absum)) in enumerate(zip(ys, refs)):
        assert y.shape == (B, Rs[i])
        assert_within(host_bf16(y), yref, absum, f"two per step {Rs} matrix {i}")


@pytest.mark.parametrize("R,B", [(16384, 8), (16377, 6)])
def test_tile_swiglu_two_tiles_per_step(R, B):
    """Gated MLP with two 16-row tiles (gate and up rows i..i+15) per step."""
    say("tile swiglu two per step", R, B)
    K = 1024
    n = oracle.col_norm(synth.calib_acts(K, 39, R))
    Wg, Wu = synth.weights(R, K, 39, 1, R), synth.weights(R, K, 39, 2, R)
    gm, gv = oracle.prune_pack(Wg, n, 8, 16)
    um, uv = oracle.prune_pack(Wu, n, 8, 16)
    x = synth.decode_x(B, K, 39, R, B)
    h = host_bf16(nm.nm_spmv_swiglu((dev_u32(gm), dev_bf16(gv)), (dev_u32(um), dev_bf16(uv)), dev_bf16(x)))
    g, ag = oracle.spmv(gm, gv, x, K, nthreads=8)
    u, au = oracle.spmv(um, uv, x, K, nthreads=8)
    ref = oracle.swiglu(g, u)
    ok = np.abs(bf16_as_f64(h) - ref) <= oracle.swiglu_tolerance(g, ag, u, au)
    assert ok.all(), f"swiglu two per step R={R} B={B}: {int((~ok).sum())} outside"


# B = 3 or 4 with K above 10240 columns (a row's x exceeds the word-per-lane kernel's
# LDS slice) and at least 512 rows: these launches run on the tile path too.
@pytest.mark.parametrize("R,K,B", [(4096, 14336, 4), (1000, 11264, 3), (513, 12288, 4), (2048, 28672, 3)])
def test_tile_small_batch_wide_rows(R, K, B):
    assert nm.nm_spmv_plan(R, K, B)["kernel"] == nm.NM_KERNEL_TILE
    say("tile small batch wide", R, K, B)
    W = synth.weights(R, K, 40, R, K, B)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 40, R)), 8, 16)
    x = synth.decode_x(B, K, 40, R, K, B)
    y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=8)
    assert_within(host_bf16(y), yref, absum, f"tile R={R} K={K} B={B}")


@pytest.mark.parametrize("B", [3, 4])
def test_tile_small_batch_multi_and_swiglu(B):
    say("tile small batch multi+swiglu", B)
    K = 11264
    x = synth.decode_x(B, K, 41, B)
    n = oracle.col_norm(synth.calib_acts(K, 41, B))
    packed, refs = [], []
    for i, R in enumerate([512, 256, 250]):
        mref, vref = oracle.prune_pack(synth.weights(R, K, 41, B, i), n, 2, 4)
        refs.append(oracle.spmv(mref, vref, x, K, nthreads=8))
        packed.append((dev_u32(mref), dev_bf16(vref)))
    ys = nm.nm_spmv_multi(packed, dev_bf16(x))
    for i, (y, (yref, absum)) in enumerate(zip(ys, refs)):
        assert_within(host_bf16(y), yref, absum, f"multi B={B} matrix {i}")
    R = 600
    gm, gv = oracle.prune_pack(synth.weights(R, K, 41, B, 10), n, 4, 8)
    um, uv = oracle.prune_pack(synth.weights(R, K, 41, B, 11), n, 4, 8)
    h = host_bf16(nm.nm_spmv_swiglu((dev_u32(gm), dev_bf16(gv)), (dev_u32(um), dev_bf16(uv)), dev_bf16(x)))
    g, ag = oracle.spmv(gm, gv, x, K, nthreads=8)
    u, au = oracle.spmv(um, uv, x, K, nthreads=8)
    ok = np.abs(bf16_as_f64(h) - oracle.swiglu(g, u)) <= oracle.swiglu_tolerance(g, ag, u, au)
    assert ok.all(), f"swiglu B={B}: {int((~ok).sum())} outside"


# Shapes where every wave keeps its x operand in registers for the whole launch (exactly
# four steps per wave and unit: K = 4096 with 8-wave workgroups, 8192 with 16-wave ones),
# with more units than workgroups and with two tiles per step, beside shapes that re-read
# x every step.  Integer-valued operands, so the result must equal the oracle exactly.
# xreg None: the planner may take either walk.
XREG = [(300, 4096, 8, 4), (9000, 4096, 5, 4), (1000, 8192, 8, 4), (5000, 8192, 6, 4), (9000, 8192, 7, None),
        (300, 2048, 6, 0), (3000, 14336, 8, 0)]


@pytest.mark.parametrize("R,K,B,xreg", XREG)
def test_tile_x_in_registers_integer_exact(R, K, B, xreg):
    say("tile x in registers", R, K, B)
    plan = nm.nm_spmv_plan(R, K, B)
    assert plan["kernel"] == nm.NM_KERNEL_TILE
    if xreg is not None:
        assert plan["x_steps_in_registers"] == xreg
    W = synth.ternary((R, K), 44, R, K, B)
    x = synth.ternary_sparse((B, K), 1024 / K, 45, R, K, B)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 44, R)), 8, 16)
    y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    yref, _ = oracle.spmv(mref, vref, x, K, nthreads=8)
    assert np.abs(yref).max() <= 256
    got = bf16_as_f64(host_bf16(y))
    assert (got == yref).all(), f"{int((got != yref).sum())} of {got.size} differ"


def test_tile_x_in_registers_two_tiles_swiglu():
    """Gated MLP, 16384 rows each, K = 4096, 8 tokens: two tiles per step, x in registers."""
    R, K, B = 16384, 4096, 8
    say("tile x in registers swiglu", R, K, B)
    plan = nm.nm_spmv_plan(R, K, B, nm.NM_EPI_SWIGLU)
    assert (plan["kernel"], plan["tiles_per_step"], plan["x_steps_in_registers"]) == (nm.NM_KERNEL_TILE, 2, 4)
    n = oracle.col_norm(synth.calib_acts(K, 46, R))
    Wg, Wu = synth.weights(R, K, 46, 1), synth.weights(R, K, 46, 2)
    gm, gv = oracle.prune_pack(Wg, n, 2, 4)
    um, uv = oracle.prune_pack(Wu, n, 2, 4)
    x = synth.decode_x(B, K, 46, B)
    h = host_bf16(nm.nm_spmv_swiglu((dev_u32(gm), dev_bf16(gv)), (dev_u32(um), dev_bf16(uv)), dev_bf16(x)))
    g, ag = oracle.spmv(gm, gv, x, K, nthreads=8)
    u, au = oracle.spmv(um, uv, x, K, nthreads=8)
    ref = oracle.swiglu(g, u)
    ok = np.abs(bf16_as_f64(h) - ref) <= oracle.swiglu_tolerance(g, ag, u, au)
    assert ok.all(), f"swiglu x in registers: {int((~ok).sum())} outside"
