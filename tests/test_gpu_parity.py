"""GPU parity: the HIP path (through the C ABI, via the thin binding) against the CPU
oracle on the same seeded inputs.

Bars: bit-exact column norms, masks, packed values and unpacked matrices; SpMV and
GEMV outputs within |y - y_ref| <= 1e-2 |y_ref| + 1e-3 sum_j |W_ij x_j| element by
element; exact equality where the result is an integer or a power-of-two rescaling.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import pins
from tests.gpu_util import (bf16_as_f64, dev_bf16, dev_f32, dev_u32, host_bf16, host_f32, host_u32, say)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402  (fails loudly if the library is missing)

PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]
RTOL, ATOL_FRAC = 1e-2, 1e-3


def assert_within(y_gpu_bits, y_ref, absum, what):
    y = bf16_as_f64(y_gpu_bits)
    ok = oracle.within_tolerance(y, y_ref, absum, RTOL, ATOL_FRAC)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance, e.g. "
                             + ", ".join(f"{tuple(i)}: gpu={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r}" for i in idx))


def gpu_pack(W_bits, X_bits, N, M):
    n = nm.nm_col_norm(dev_bf16(X_bits))
    masks, values = nm.nm_prune_pack(dev_bf16(W_bits), n, N, M)
    torch.cuda.synchronize()
    return host_f32(n), host_u32(masks), host_bf16(values), masks, values


# ------------------------------------------------------------------ column norm
@pytest.mark.parametrize("T,K", [(16, 512), (16, 4096), (7, 1000), (1, 33), (16, 28672)])
def test_col_norm_bit_exact(T, K):
    say("col_norm", T, K)
    X = synth.calib_acts(K, 0, T, K, T=T)
    got = host_f32(nm.nm_col_norm(dev_bf16(X)))
    ref = oracle.col_norm(X)
    assert (got.view(np.uint32) == ref.view(np.uint32)).all()


def test_col_norm_closed_forms_and_tiny_values():
    say("col_norm closed forms")
    X = np.zeros((16, 64), np.float32)
    X[0, 0], X[1, 0] = 3.0, 4.0
    X[:, 1] = -3.0
    X[5, 3] = -2.0 ** -100
    X[2, 5] = 2.0 ** -130  # bf16 subnormal input
    Xb = synth.to_bf16_bits(X)
    got = host_f32(nm.nm_col_norm(dev_bf16(Xb)))
    assert got[0] == 5.0 and got[1] == 12.0 and got[2] == 0.0 and got[3] == 2.0 ** -100
    assert (got.view(np.uint32) == oracle.col_norm(Xb).view(np.uint32)).all()


# ------------------------------------------------------------------ select + pack
@pytest.mark.parametrize("N,M", PATTERNS)
@pytest.mark.parametrize("R,K", [(256, 512), (37, 1024), (1, 32), (300, 4096)])
def test_prune_pack_bit_exact(N, M, R, K):
    say("prune_pack", N, M, R, K)
    W = synth.weights(R, K, 1, R, K, M)
    X = synth.calib_acts(K, 1, R, K, M)
    n, m, v, _, _ = gpu_pack(W, X, N, M)
    nref = oracle.col_norm(X)
    mref, vref = oracle.prune_pack(W, nref, N, M)
    assert (n.view(np.uint32) == nref.view(np.uint32)).all()
    assert (m == mref).all()
    assert (v == vref).all()
    assert pins.certificate_ok(W, n, m, N, M).all()


@pytest.mark.parametrize("N,M", PATTERNS)
def test_prune_pack_tie_stress_and_signed_zero(N, M):
    say("prune_pack ties", N, M)
    R, K = 64, 1024
    W, n = synth.tie_stress(R, K, 2, M)
    masks, values = nm.nm_prune_pack(dev_bf16(W), dev_f32(n), N, M)
    mref, vref = oracle.prune_pack(W, n, N, M)
    assert (host_u32(masks) == mref).all()
    assert (host_bf16(values) == vref).all()


def test_prune_pack_subnormal_weights_and_norms():
    """Exact scores must not flush: tiny bf16 weights and fp32 subnormal norms."""
    say("prune_pack subnormal")
    R, K = 8, 256
    g = synth.rng(3, 3)
    W = synth.to_bf16_bits((g.standard_normal((R, K)) * 2.0 ** -128).astype(np.float32))
    n = (g.random(K) * 2.0 ** -140).astype(np.float32)
    n[::5] = np.float32(1e-45)
    masks, values = nm.nm_prune_pack(dev_bf16(W), dev_f32(n), 4, 8)
    mref, vref = oracle.prune_pack(W, n, 4, 8)
    assert (host_u32(masks) == mref).all() and (host_bf16(values) == vref).all()


def test_prune_pack_strided_input():
    say("prune_pack strided W")
    R, K, ld = 48, 512, 640
    Wfull = synth.weights(R, ld, 4)
    X = synth.calib_acts(K, 4)
    Wd = dev_bf16(Wfull)[:, :K]
    n = nm.nm_col_norm(dev_bf16(X))
    masks, values = nm.nm_prune_pack(Wd, n, 8, 16)
    mref, vref = oracle.prune_pack(np.ascontiguousarray(Wfull[:, :K]), oracle.col_norm(X), 8, 16)
    assert (host_u32(masks) == mref).all() and (host_bf16(values) == vref).all()


# ------------------------------------------------------------------ unpack
@pytest.mark.parametrize("N,M", [(2, 4), (16, 32)])
def test_unpack_bit_exact(N, M):
    say("unpack", N, M)
    R, K = 200, 2048
    W = synth.weights(R, K, 5)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 5)), N, M)
    Wp = nm.nm_unpack(dev_u32(mref), dev_bf16(vref))
    assert (host_bf16(Wp) == oracle.unpack(mref, vref, K)).all()


# ------------------------------------------------------------------ SpMV
SPMV_SHAPES = [
    (256, 512),     # tiny workload shape
    (1000, 4096),   # ragged row count (not a multiple of the 8 waves per workgroup)
    (1024, 4096),   # k/v 8B shape
    (513, 5120),    # words per row not a multiple of 64
    (96, 14336),    # long rows (down projection shape)
    (17, 8192),     # few rows: rows split into slices (workspace + second pass)
    (1, 32),        # smallest legal matrix
    (3, 28672),     # longest rows, x = 56 KB
]


@pytest.mark.parametrize("R,K", SPMV_SHAPES)
@pytest.mark.parametrize("B", [1, 2, 8])
def test_spmv_within_tolerance(R, K, B):
    say("spmv", R, K, B)
    M = 8
    W = synth.weights(R, K, 6, R, K)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 6, R, K)), M // 2, M)
    x = synth.decode_x(B, K, 6, R, K, B)
    y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    torch.cuda.synchronize()
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=4)
    assert_within(host_bf16(y), yref, absum, f"spmv R={R} K={K} B={B}")


@pytest.mark.parametrize("B", [2, 3, 4, 5, 8])
def test_spmv_word_walk_ragged_strips(B):
    # 4160 columns = 130 words: two whole 64-word strips and a 2-word strip, and K is no
    # multiple of 1024, so every B takes the word-per-lane walk (x in whole strips of LDS
    # panels at B >= 2, the last one mostly unused).  600 rows keep whole rows in one
    # slice up to four tokens (at 5-8 tokens the x of 130 words exceeds one slice: slices
    # of 128 and 2 words); 9 rows are cut into the same two slices to spread the work.
    say("spmv ragged strips", B)
    for R, splits in ((600, 1 if B <= 4 else 2), (9, 2)):
        p = nm.nm_spmv_plan(R, 4160, B)
        assert p["kernel"] == 0 and p["splits"] == splits, p
        W = synth.weights(R, 4160, 23, R, B)
        mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(4160, 23, R)), 4, 8)
        x = synth.decode_x(B, 4160, 23, R, B)
        y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
        yref, absum = oracle.spmv(mref, vref, x, 4160, nthreads=4)
        assert_within(host_bf16(y), yref, absum, f"spmv ragged strips R={R} B={B}")


@pytest.mark.parametrize("B", [3, 4, 5, 6, 7])
def test_spmv_every_batch_size(B):
    say("spmv batch", B)
    R, K = 384, 8192
    W = synth.weights(R, K, 7, B)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 7, B)), 16, 32)
    x = synth.decode_x(B, K, 7, B)
    y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=4)
    assert_within(host_bf16(y), yref, absum, f"spmv B={B}")


# Shapes that reach the planner's larger launch forms, each with the plan it must get
# (kernel: 0 word-per-lane, 1 matrix-core tile; workgroup size; row slices), so a planner
# change that moves a shape to another kernel instance fails here instead of silently
# dropping that instance from the parity tests:
# * 1024-thread word-per-lane workgroups at B = 3/4 (x allows only two workgroups per CU)
#   and at B = 1/2 for rows of 8192+ columns that split evenly over waves and CUs;
# * split rows with 1024 threads (B = 2, K = 28672) and 256-thread workgroups for few rows;
# * the tile kernel at B = 3/4 where a row's x exceeds the word-per-lane LDS slice.
WIDE = [(3000, 8192, 3, (0, 1024, 1)), (2100, 8192, 4, (0, 1024, 1)), (4096, 8192, 1, (0, 1024, 1)),
        (4096, 16384, 2, (0, 1024, 1)), (2048, 28672, 2, (0, 1024, 2)), (1000, 28672, 1, (0, 256, 1)),
        (300, 28672, 3, (0, 256, 3)), (1024, 8192, 1, (0, 256, 1)), (700, 28672, 4, (1, 1024, 1)),
        (2049, 11264, 3, (1, 512, 1))]


@pytest.mark.parametrize("R,K,B,plan", WIDE)
def test_spmv_wide_workgroups(R, K, B, plan):
    p = nm.nm_spmv_plan(R, K, B)
    say("spmv wide", R, K, B, p)
    assert (p["kernel"], p["threads"], p["splits"]) == plan
    W = synth.weights(R, K, 21, R, K, B)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 21, R, K)), 8, 16)
    x = synth.decode_x(B, K, 21, R, K, B)
    md, vd, xd = dev_u32(mref), dev_bf16(vref), dev_bf16(x)
    y = nm.nm_spmv(md, vd, xd)
    y2 = nm.nm_spmv(md, vd, xd)
    ys = nm.nm_spmv_multi([(md, vd), (md[: R // 3], vd[: R // 3])], xd)
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=4)
    assert_within(host_bf16(y), yref, absum, f"spmv wide R={R} K={K} B={B}")
    assert (host_bf16(y) == host_bf16(y2)).all()
    assert_within(host_bf16(ys[0]), yref, absum, "multi matrix 0")
    assert_within(host_bf16(ys[1]), yref[:, : R // 3], absum[:, : R // 3], "multi matrix 1")
    # the dense baseline takes its own larger workgroups on the same shapes
    yd = nm.dense_gemv(dev_bf16(W), xd)
    ydref, adabs = oracle.dense(W, x, nthreads=4)
    assert_within(host_bf16(yd), ydref, adabs, f"dense wide R={R} K={K} B={B}")


# One token, one matrix, rows of 7+ strips of 64 words and at least 4096 of them: each row
# is split between two waves of a 16-wave workgroup (the half-row walk), whose totals
# meet in LDS.  Ragged last workgroup (4097 rows), a ragged last strip (K = 17408: 8.5
# strips per row), every pattern, integer-exact and random data, repeat runs identical,
# a one-matrix nm_spmv_multi identical to nm_spmv, and the plan at the boundaries.
HALF = [(4096, 14336, 2, 4), (8192, 14336, 16, 32), (4096, 28672, 4, 8)]
# (rows, columns, pattern, workgroup size, rows per workgroup)
STRIPS = [(4097, 14336, 8, 16, 1024, 9), (5000, 17408, 16, 32, 1024, 10), (5120, 25600, 2, 4, 1024, 10),
          (8192, 8192, 4, 8, 512, 8), (8193, 8192, 2, 4, 512, 9), (9000, 12288, 16, 32, 512, 9)]


def _check_one_token_walk(R, K, N, M, what):
    """One-token launch of a single matrix against the oracle: ternary integer inputs
    exactly, random inputs within tolerance; repeats bit-identical; the same matrix cut
    into two nm_spmv_multi matrices (which the planner gives whole rows per wave) within
    tolerance."""
    n = oracle.col_norm(synth.calib_acts(K, 62, R, K))
    # integer-valued operands: the result equals the oracle exactly
    Wt = synth.ternary((R, K), 62, R, K)
    xt = synth.ternary_sparse((1, K), 1024 / K, 63, R, K)
    mt, vt = oracle.prune_pack(Wt, n, N, M)
    yt = host_bf16(nm.nm_spmv(dev_u32(mt), dev_bf16(vt), dev_bf16(xt)))
    ytref, _ = oracle.spmv(mt, vt, xt, K, nthreads=8)
    assert np.abs(ytref).max() <= 256
    got = bf16_as_f64(yt)
    assert (got == ytref).all(), f"{int((got != ytref).sum())} of {got.size} differ"
    # random data within tolerance; repeats and the one-matrix multi launch identical
    W = synth.weights(R, K, 64, R, K)
    mref, vref = oracle.prune_pack(W, n, N, M)
    x = synth.decode_x(1, K, 64, R, K)
    md, vd, xd = dev_u32(mref), dev_bf16(vref), dev_bf16(x)
    y = nm.nm_spmv(md, vd, xd)
    y2 = nm.nm_spmv(md, vd, xd)
    h = R // 2
    assert nm.nm_spmv_multi_plan([h, R - h], K, 1)["kernel"] == nm.NM_KERNEL_WORD
    ym = torch.cat(nm.nm_spmv_multi([(md[:h], vd[:h]), (md[h:], vd[h:])], xd), dim=1)
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=8)
    assert_within(host_bf16(y), yref, absum, f"{what} R={R} K={K} {N}:{M}")
    assert_within(host_bf16(ym), yref, absum, f"{what} (whole rows) R={R} K={K} {N}:{M}")
    assert (host_bf16(y) == host_bf16(y2)).all()


@pytest.mark.parametrize("R,K,N,M", HALF)
def test_spmv_half_rows(R, K, N, M):
    p = nm.nm_spmv_plan(R, K, 1)
    say("spmv half rows", R, K, N, M, p)
    assert (p["kernel"], p["threads"], p["grid_x"], p["splits"]) == (nm.NM_KERNEL_WORD_HALF_ROWS, 1024, (R + 7) // 8, 1)
    _check_one_token_walk(R, K, N, M, "half rows")


@pytest.mark.parametrize("R,K,N,M,nt,rpw", STRIPS)
def test_spmv_strips(R, K, N, M, nt, rpw):
    """The strip walk: consecutive rows per workgroup, strips dealt to the waves in turn,
    ragged last workgroups (R not a multiple of the rows per workgroup) included."""
    p = nm.nm_spmv_plan(R, K, 1)
    say("spmv strips", R, K, N, M, p)
    assert (p["kernel"], p["threads"], p["rows_per_group"], p["splits"]) == (nm.NM_KERNEL_WORD_STRIPS, nt, rpw, 1)
    assert p["grid_x"] == (R + rpw - 1) // rpw
    _check_one_token_walk(R, K, N, M, "strips")


def test_spmv_one_token_walk_plan_boundaries():
    """Half rows and strips are taken only at one token and one matrix: half rows for
    7+ strips per row on whole rounds of 4096 rows (on 256 CUs; the GPU here may have
    another count, so the row counts scale with it), strips for other row counts from
    16 per CU and for rows of 4-6 strips with 4+ strips per wave; other shapes keep the
    whole-row walk."""
    say("spmv one-token walk plan boundaries")
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    rnd = 2 * cu * 8
    assert nm.nm_spmv_plan(rnd, 14336, 1)["kernel"] == nm.NM_KERNEL_WORD_HALF_ROWS
    assert nm.nm_spmv_plan(rnd + 64, 14336, 1)["kernel"] == nm.NM_KERNEL_WORD_STRIPS
    assert nm.nm_spmv_plan(rnd - 1, 14336, 1)["kernel"] == nm.NM_KERNEL_WORD
    assert nm.nm_spmv_plan(rnd, 12288, 1)["kernel"] == nm.NM_KERNEL_WORD  # 6 strips, 4 per wave: no
    assert nm.nm_spmv_plan(2 * rnd, 12288, 1)["kernel"] == nm.NM_KERNEL_WORD_STRIPS
    assert nm.nm_spmv_plan(4 * cu * 8, 4096, 1)["kernel"] == nm.NM_KERNEL_WORD  # rows of 2 strips
    assert nm.nm_spmv_plan(rnd, 14336, 2)["kernel"] == nm.NM_KERNEL_WORD
    assert nm.nm_spmv_plan(2 * rnd, 8192, 2)["kernel"] == nm.NM_KERNEL_WORD
    assert nm.nm_spmv_plan(rnd, 14336, 1, nm.NM_EPI_SWIGLU)["kernel"] == nm.NM_KERNEL_WORD
    assert nm.nm_spmv_multi_plan([rnd // 2, rnd // 2], 14336, 1)["kernel"] == nm.NM_KERNEL_WORD


@pytest.mark.parametrize("N,M", PATTERNS)
def test_spmv_integer_exact(N, M):
    """Ternary weights and inputs: every partial sum is an integer <= K/2 in
    magnitude, exact in fp32 and representable in bf16 up to 256, so the GPU result
    must equal the oracle's bit for bit whatever the summation order."""
    say("spmv integer exact", N, M)
    R, K, B = 300, 512, 4
    W = synth.ternary((R, K), 8, M)
    x = synth.ternary((B, K), 9, M)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 8)), N, M)
    y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    yref, _ = oracle.spmv(mref, vref, x, K)
    assert np.abs(yref).max() <= 256
    assert (bf16_as_f64(host_bf16(y)) == yref).all()


# 6 tokens: the matrix-core walk; 2-4 tokens: the word walk, whose row totals of the
# tokens are reduced together and stored by one lane per token (a token routed to the
# wrong output row, or a column of another lane's block, shows here exactly).
@pytest.mark.parametrize("cols", [[0, 1, 31, 32, 2047, 4095], [33, 4095], [0, 2047, 4064], [5, 1000, 31, 4090]])
def test_spmv_one_hot_reads_columns(cols):
    say("spmv one-hot", cols)
    R, K = 512, 4096
    W = synth.weights(R, K, 10)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 10)), 2, 4)
    Wp = oracle.unpack(mref, vref, K)
    x = np.zeros((len(cols), K), np.uint16)
    for b, j in enumerate(cols):
        x[b, j] = 0x3F80
    y = host_bf16(nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x)))
    for b, j in enumerate(cols):
        assert (y[b] == Wp[:, j]).all()


@pytest.mark.parametrize("B", [1, 2, 4])
def test_spmv_power_of_two_scaling_and_determinism(B):
    say("spmv scaling + determinism", B)
    R, K = 2048, 4096
    W = synth.weights(R, K, 11)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 11)), 4, 8)
    m, v = dev_u32(mref), dev_bf16(vref)
    x = synth.decode_x(B, K, 11)
    x4 = synth.to_bf16_bits(synth.bf16_bits_to_f32(x) * 4.0)
    y1 = host_bf16(nm.nm_spmv(m, v, dev_bf16(x)))
    y1b = host_bf16(nm.nm_spmv(m, v, dev_bf16(x)))
    y4 = host_bf16(nm.nm_spmv(m, v, dev_bf16(x4)))
    assert (y1 == y1b).all()  # run-to-run bit reproducibility (no atomics)
    assert (bf16_as_f64(y4) == 4.0 * bf16_as_f64(y1)).all()


def test_spmv_pattern_agnostic_kernel():
    """Same bytes, four patterns: each result matches its own oracle."""
    R, K = 640, 4096
    W = synth.weights(R, K, 12)
    n = oracle.col_norm(synth.calib_acts(K, 12))
    x = synth.decode_x(1, K, 12)
    for N, M in PATTERNS:
        say("spmv pattern", N, M)
        mref, vref = oracle.prune_pack(W, n, N, M)
        y = nm.nm_spmv(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
        yref, absum = oracle.spmv(mref, vref, x, K)
        assert_within(host_bf16(y), yref, absum, f"{N}:{M}")


def test_spmv_strided_x_and_y():
    say("spmv strided x/y")
    R, K, B = 700, 4096, 3
    W = synth.weights(R, K, 13)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 13)), 2, 4)
    xfull = synth.decode_x(B, K + 64, 13)
    xd = dev_bf16(xfull)[:, :K]
    yfull = torch.zeros((B, R + 40), dtype=torch.bfloat16, device="cuda")
    nm.nm_spmv(dev_u32(mref), dev_bf16(vref), xd, out=yfull[:, :R])
    yh = host_bf16(yfull)
    yref, absum = oracle.spmv(mref, vref, np.ascontiguousarray(xfull[:, :K]), K)
    assert_within(yh[:, :R], yref, absum, "strided")
    assert (yh[:, R:] == 0).all()  # nothing written past ldy's row


# Mask words without exactly 16 set bits are outside the input contract: every walk then
# reads fixed columns of the word's own block (no access outside the staged x or the
# dense tile), so the other rows of the launch are unaffected and every output is finite.
BAD_WORDS = [(3, 5, 0x00000000), (77, 40, 0xFFFFFFFF), (150, 100, 0x00010001), (299, 127, 0x7FFFFFFF)]


@pytest.mark.parametrize("R,K,B", [(300, 4096, 1), (300, 4096, 2), (300, 4096, 4), (300, 4096, 8),
                                   (4096, 14336, 1)])
def test_spmv_malformed_mask_words_stay_in_their_rows(R, K, B):
    say("spmv malformed words", R, K, B)
    W = synth.weights(R, K, 14, R, K)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 14, R)), 4, 8)
    bad = mref.copy()
    rows = sorted({r for r, _, _ in BAD_WORDS if r < R})
    for r, w, word in BAD_WORDS:
        if r < R:
            bad[r, w] = word
    x = synth.decode_x(B, K, 14, R, K, B)
    y = bf16_as_f64(host_bf16(nm.nm_spmv(dev_u32(bad), dev_bf16(vref), dev_bf16(x))))
    assert np.isfinite(y).all()
    yref, absum = oracle.spmv(mref, vref, x, K, nthreads=8)
    keep = np.setdiff1d(np.arange(R), rows)
    ok = oracle.within_tolerance(y[:, keep], yref[:, keep], absum[:, keep], RTOL, ATOL_FRAC)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} rows outside tolerance next to malformed words"


def test_spmv_workspace_errors():
    say("spmv workspace errors")
    R, K = 64, 8192
    need = nm.nm_spmv_workspace_bytes(R, K, 1)
    assert need > 0  # so few rows that each row is split across workgroups
    m = torch.zeros((R, K // 32), dtype=torch.int32, device="cuda")
    v = torch.zeros((R, K // 2), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((1, K), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(need // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(nm.NmError) as e:
        nm.nm_spmv(m, v, x, workspace=small)
    assert e.value.status == 5


# ------------------------------------------------------------------ dense GEMV
@pytest.mark.parametrize("R,K", [(256, 512), (1000, 4096), (96, 14336), (5, 28672), (1, 8), (77, 1000)])
@pytest.mark.parametrize("B", [1, 4, 8])
def test_dense_within_tolerance(R, K, B):
    say("dense", R, K, B)
    W = synth.weights(R, K, 14, R, K)
    x = synth.decode_x(B, K, 14, R, K, B)
    y = nm.dense_gemv(dev_bf16(W), dev_bf16(x))
    yref, absum = oracle.dense(W, x, nthreads=4)
    assert_within(host_bf16(y), yref, absum, f"dense R={R} K={K} B={B}")


def test_dense_integer_exact():
    say("dense integer exact")
    R, K, B = 200, 256, 2
    W = synth.ternary((R, K), 15)
    x = synth.ternary((B, K), 16)
    y = nm.dense_gemv(dev_bf16(W), dev_bf16(x))
    yref, _ = oracle.dense(W, x)
    assert (bf16_as_f64(host_bf16(y)) == yref).all()


def test_sparse_equals_dense_of_unpacked():
    say("spmv vs dense(unpack)")
    R, K = 1536, 4096
    W = synth.weights(R, K, 17)
    X = synth.calib_acts(K, 17)
    x = synth.decode_x(1, K, 17)
    n = nm.nm_col_norm(dev_bf16(X))
    masks, values = nm.nm_prune_pack(dev_bf16(W), n, 8, 16)
    ys = host_bf16(nm.nm_spmv(masks, values, dev_bf16(x)))
    yd = host_bf16(nm.dense_gemv(nm.nm_unpack(masks, values), dev_bf16(x)))
    mref, vref = oracle.prune_pack(W, oracle.col_norm(X), 8, 16)
    yref, absum = oracle.spmv(mref, vref, x, K)
    assert_within(ys, yref, absum, "sparse")
    assert_within(yd, yref, absum, "dense of unpacked")


# ------------------------------------------------------------------ several matrices, one launch
@pytest.mark.parametrize("B", [1, 4])
def test_spmv_multi_matches_oracle_and_separate_calls(B):
    say("spmv multi", B)
    K = 4096
    Rs = [640, 520, 1000]  # q/k/v-like group with ragged row counts
    x = synth.decode_x(B, K, 18, B)
    n = oracle.col_norm(synth.calib_acts(K, 18))
    refs, packed = [], []
    for i, R in enumerate(Rs):
        W = synth.weights(R, K, 18, i)
        mref, vref = oracle.prune_pack(W, n, 8, 16)
        refs.append(oracle.spmv(mref, vref, x, K, nthreads=4))
        packed.append((dev_u32(mref), dev_bf16(vref)))
    xd = dev_bf16(x)
    ys = nm.nm_spmv_multi(packed, xd)
    singles = [nm.nm_spmv(m, v, xd) for m, v in packed]
    for i, (y, (yref, absum)) in enumerate(zip(ys, refs)):
        assert_within(host_bf16(y), yref, absum, f"multi matrix {i}")
        # every matrix has >= 512 rows, so neither launch splits rows: identical arithmetic
        assert (host_bf16(y) == host_bf16(singles[i])).all()


def test_spmv_multi_split_rows_and_single_matrix():
    say("spmv multi split rows")
    K = 8192
    Rs = [7, 33]
    x = synth.decode_x(2, K, 19)
    packed, refs = [], []
    for i, R in enumerate(Rs):
        W = synth.weights(R, K, 19, i)
        mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 19, i)), 2, 4)
        refs.append(oracle.spmv(mref, vref, x, K))
        packed.append((dev_u32(mref), dev_bf16(vref)))
    assert nm.nm_spmv_multi_workspace_bytes(Rs, K, 2) > 0
    ys = nm.nm_spmv_multi(packed, dev_bf16(x))
    for i, (y, (yref, absum)) in enumerate(zip(ys, refs)):
        assert_within(host_bf16(y), yref, absum, f"split multi {i}")
    y1 = nm.nm_spmv_multi(packed[:1], dev_bf16(x))[0]
    assert_within(host_bf16(y1), *refs[0], "single-matrix multi")


@pytest.mark.parametrize("P", [7, 8])
def test_spmv_multi_many_ragged_matrices(P):
    """Up to the maximum of eight matrices per launch, with ragged row counts (1 row,
    fewer rows than a workgroup's waves, rows not a multiple of 8): every launch row is
    attributed to its own matrix and written to that matrix's output."""
    say("spmv multi many", P)
    K, B = 1024, 3
    Rs = [5, 64, 1, 300, 17, 8, 129, 2][:P]
    x = synth.decode_x(B, K, 20, P)
    n = oracle.col_norm(synth.calib_acts(K, 20, P))
    packed, refs = [], []
    for i, R in enumerate(Rs):
        W = synth.weights(R, K, 20, P, i)
        mref, vref = oracle.prune_pack(W, n, 4, 8)
        refs.append(oracle.spmv(mref, vref, x, K))
        packed.append((dev_u32(mref), dev_bf16(vref)))
    ys = nm.nm_spmv_multi(packed, dev_bf16(x))
    for i, (y, (yref, absum)) in enumerate(zip(ys, refs)):
        assert y.shape == (B, Rs[i])
        assert_within(host_bf16(y), yref, absum, f"multi P={P} matrix {i}")


@pytest.mark.parametrize("B", [1, 8])
def test_dense_multi_matches_oracle(B):
    say("dense multi", B)
    K = 4096
    Rs = [700, 96, 1500]
    x = synth.decode_x(B, K, 20, B)
    Ws = [synth.weights(R, K, 20, i) for i, R in enumerate(Rs)]
    ys = nm.dense_gemv_multi([dev_bf16(W) for W in Ws], dev_bf16(x))
    for i, (y, W) in enumerate(zip(ys, Ws)):
        yref, absum = oracle.dense(W, x, nthreads=4)
        assert_within(host_bf16(y), yref, absum, f"dense multi {i}")
