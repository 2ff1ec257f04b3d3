"""Pins for the CPU oracle: each oracle function is tied to something other than
itself -- a hand-worked fixture, the pages' stated invariants and closed forms,
brute force on tiny inputs, exact rational arithmetic, and numpy's library
matmul -- and the mutation tests show that a plausible mistake planted in the
oracle's output is caught by at least one of those pins.
"""
from __future__ import annotations

import os
import numpy as np
import pytest

import oracle
import synth
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]


# ------------------------------------------------------------------ fixtures
def _load_worked():
    W = n = None
    keep, mask, values, y_ones = {}, {}, {}, {}
    with open(os.path.join(GOLDEN, "worked_row_k32.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *rest = line.split()
            if tag == "W":
                W = np.array([float(v) for v in rest], dtype=np.float32)
            elif tag == "n":
                n = np.array([float(v) for v in rest], dtype=np.float32)
            elif tag == "keep":
                keep[rest[0]] = [int(v) for v in rest[1:]]
            elif tag == "mask":
                mask[rest[0]] = int(rest[1], 16)
            elif tag == "values":
                values[rest[0]] = [int(v, 16) for v in rest[1:]]
            elif tag == "y_ones":
                y_ones[rest[0]] = float(rest[1])
    return W, n, keep, mask, values, y_ones


def test_worked_example_by_hand():
    W, n, keep, mask, values, y_ones = _load_worked()
    Wb = synth.to_bf16_bits(W)[None, :]
    # -0.0 must keep its sign bit in the input
    assert Wb[0, 4] == 0x8000
    for pat in ("2:4", "4:8", "8:16", "16:32"):
        N, M = (int(v) for v in pat.split(":"))
        m, v = oracle.prune_pack(Wb, n, N, M)
        assert int(m[0, 0]) == mask[pat], pat
        got = [c for c in range(32) if (int(m[0, 0]) >> c) & 1]
        assert got == keep[pat], pat
        assert [int(t) for t in v[0]] == [int(Wb[0, c]) for c in keep[pat]]
    m, v = oracle.prune_pack(Wb, n, 2, 4)
    assert [int(t) for t in v[0]] == values["2:4"]
    ones = synth.to_bf16_bits(np.ones((1, 32), np.float32))
    y, a = oracle.spmv(m, v, ones, 32)
    assert y[0, 0] == y_ones["2:4"]
    yd, _ = oracle.dense(Wb, ones)
    assert yd[0, 0] == y_ones["dense"]


def test_metadata_closed_form():
    """Pages: 2 bits of mask per kept weight at 50%, 16x less than an int32 index and
    4x less than a uint8 offset; 16 set bits in every aligned word."""
    fx = {}
    with open(os.path.join(GOLDEN, "metadata_bits.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                fx[k] = int(v)
    R, K = 48, 256
    W = synth.weights(R, K, 7)
    n = oracle.col_norm(synth.calib_acts(K, 7))
    for N, M in PATTERNS:
        m, v = oracle.prune_pack(W, n, N, M)
        nnz = R * K // 2
        assert m.nbytes * 8 == fx["bitmask_bits_per_nnz"] * nnz
        assert m.nbytes == R * K // 8 and v.nbytes == R * K  # bf16, K/2 per row
        assert fx["int32_index_bits_per_nnz"] // fx["bitmask_bits_per_nnz"] == fx["ratio_vs_int32"]
        assert fx["uint8_offset_bits_per_nnz"] // fx["bitmask_bits_per_nnz"] == fx["ratio_vs_uint8"]
        assert (pins.popcounts(m) == fx["set_bits_per_word"]).all()


# ------------------------------------------------------------------ selection
@pytest.mark.parametrize("N,M", PATTERNS)
@pytest.mark.parametrize("seed", [0, 1])
def test_certificate_random(N, M, seed):
    R, K = 64, 512
    W = synth.weights(R, K, seed, M)
    n = oracle.col_norm(synth.calib_acts(K, seed, M))
    m, v = oracle.prune_pack(W, n, N, M)
    assert pins.certificate_ok(W, n, m, N, M).all()
    assert (pins.popcounts(m) == 16).all()
    assert (pins.pack_by_indexing(W, m) == v).all()


@pytest.mark.parametrize("N,M", PATTERNS)
def test_certificate_tie_stress(N, M):
    W, n = synth.tie_stress(32, 256, 3, M)
    m, v = oracle.prune_pack(W, n, N, M)
    ok = pins.certificate_ok(W, n, m, N, M)
    assert ok.all()
    # the tie rule really is exercised: many groups have equal scores across the cut
    s = pins.exact_scores(W, n).reshape(32, 256 // M, M)
    kept = pins.mask_bits(m, 256).reshape(s.shape)
    ks = np.where(kept, s, np.inf).min(-1)
    ds = np.where(~kept, s, -np.inf).max(-1)
    assert (ks == ds).mean() > 0.2


@pytest.mark.parametrize("N,M", [(2, 4), (4, 8), (8, 16)])
@pytest.mark.parametrize("kind", ["random", "ties"])
def test_brute_force_tiny(N, M, kind):
    R, K = 2, 64
    if kind == "random":
        W = synth.weights(R, K, 11, M)
        n = oracle.col_norm(synth.calib_acts(K, 11, M))
    else:
        W, n = synth.tie_stress(R, K, 12, M)
    m, _ = oracle.prune_pack(W, n, N, M)
    kept = pins.mask_bits(m, K)
    s = pins.exact_scores(W, n)
    for i in range(R):
        for g0 in range(0, K, M):
            best = pins.brute_force_group(s[i, g0:g0 + M], N)
            got = tuple(int(c) for c in np.nonzero(kept[i, g0:g0 + M])[0])
            assert got == best, (i, g0)


@pytest.mark.parametrize("N,M", PATTERNS)
def test_magnitude_pruning_special_case(N, M):
    """With every column norm equal to 1 the method is plain magnitude pruning: the
    kept set is numpy's stable descending sort of |W| cut at N."""
    R, K = 16, 256
    W = synth.weights(R, K, 21, M)
    W[:, ::7] = 0  # plenty of exact ties at zero
    n = np.ones(K, np.float32)
    m, _ = oracle.prune_pack(W, n, N, M)
    kept = pins.mask_bits(m, K).reshape(R, K // M, M)
    mag = np.abs(pins.bf16_to_f64(W)).reshape(R, K // M, M)
    order = np.argsort(-mag, axis=-1, kind="stable")[..., :N]
    exp = np.zeros_like(kept)
    np.put_along_axis(exp, order, True, axis=-1)
    assert (kept == exp).all()


# ------------------------------------------------------------------ encoding
@pytest.mark.parametrize("N,M", PATTERNS)
def test_roundtrip(N, M):
    R, K = 40, 320
    W = synth.weights(R, K, 31, M)
    W[3, 5] = 0x8000  # -0.0 survives as a raw pattern when kept
    n = oracle.col_norm(synth.calib_acts(K, 31, M))
    m, v = oracle.prune_pack(W, n, N, M)
    Wp = oracle.unpack(m, v, K)
    bits = pins.mask_bits(m, K)
    assert (Wp == np.where(bits, W, 0)).all()
    assert (Wp == pins.unpack_by_indexing(m, v, K)).all()
    assert (pins.pack_by_indexing(Wp, m) == v).all()


# ------------------------------------------------------------------ column norm
def test_col_norm_closed_forms():
    # 3-4-5: sqrt(9 + 16) = 5; constant column a over T tokens: |a| sqrt(T)
    X = np.zeros((16, 64), np.float32)
    X[0, 0], X[1, 0] = 3.0, 4.0
    X[:, 1] = -3.0  # 3 * 4 = 12
    X[:, 2] = 0.0
    X[5, 3] = -2.0 ** -100  # tiny values do not flush
    X[:4, 4] = 0.5  # 0.5 * 2 = 1
    n = oracle.col_norm(synth.to_bf16_bits(X))
    assert n[0] == 5.0 and n[1] == 12.0 and n[2] == 0.0 and n[3] == 2.0 ** -100 and n[4] == 1.0


def test_col_norm_exact_rational():
    """Bounded exponents make the fp64 token sum exact, so the oracle must equal the
    correctly rounded square root of the exact rational sum, rounded to fp32."""
    g = synth.rng(5, 99)
    T, K = 16, 96
    mant = g.integers(128, 256, size=(T, K)).astype(np.float64)
    expo = g.integers(-14, 8, size=(T, K))
    sign = g.choice([-1.0, 1.0], size=(T, K))
    X = synth.to_bf16_bits((sign * mant * np.exp2(expo - 7)).astype(np.float32))
    assert (oracle.col_norm(X) == pins.exact_col_norm(X)).all()


def test_col_norm_lognormal_within_one_ulp():
    X = synth.calib_acts(256, 8)
    got = oracle.col_norm(X)
    ref = pins.exact_col_norm(X)
    ulp = np.spacing(np.abs(ref))
    assert (np.abs(got - ref) <= ulp).all()
    assert (got == ref).mean() > 0.99


# ------------------------------------------------------------------ matvec
@pytest.mark.parametrize("B", [1, 3, 8])
def test_spmv_vs_numpy_matmul(B):
    R, K = 96, 640
    W = synth.weights(R, K, 41, B)
    n = oracle.col_norm(synth.calib_acts(K, 41, B))
    m, v = oracle.prune_pack(W, n, 4, 8)
    x = synth.decode_x(B, K, 41)
    y, a = oracle.spmv(m, v, x, K, nthreads=3)
    Wp = pins.bf16_to_f64(pins.unpack_by_indexing(m, v, K))
    xf = pins.bf16_to_f64(x)
    ref = xf @ Wp.T
    aref = np.abs(xf) @ np.abs(Wp).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * aref.max())
    assert np.allclose(a, aref, rtol=1e-12)
    yd, ad = oracle.dense(W, x, nthreads=2)
    assert np.allclose(yd, xf @ pins.bf16_to_f64(W).T, rtol=1e-12, atol=1e-12 * ad.max())


def test_matvec_integer_exact():
    """Ternary weights and inputs: every output is an integer; compare with Python
    integer sums (exact, any order)."""
    R, K, B = 24, 512, 2
    W = synth.ternary((R, K), 51)
    x = synth.ternary((B, K), 52)
    n = oracle.col_norm(synth.calib_acts(K, 53))
    m, v = oracle.prune_pack(W, n, 8, 16)
    Wp = pins.unpack_by_indexing(m, v, K)
    wi = pins.bf16_to_f64(Wp).astype(np.int64)
    xi = pins.bf16_to_f64(x).astype(np.int64)
    y, _ = oracle.spmv(m, v, x, K)
    for b in range(B):
        for i in range(R):
            assert y[b, i] == sum(int(p) * int(q) for p, q in zip(wi[i], xi[b]))
    yd, _ = oracle.dense(W, x)
    wd = pins.bf16_to_f64(W).astype(np.int64)
    assert (yd == (xi @ wd.T).astype(np.float64)).all()


def test_spmv_one_hot_reads_a_column():
    R, K = 32, 256
    W = synth.weights(R, K, 61)
    n = oracle.col_norm(synth.calib_acts(K, 61))
    m, v = oracle.prune_pack(W, n, 16, 32)
    Wp = pins.unpack_by_indexing(m, v, K)
    for j in (0, 1, 31, 32, 255):
        x = np.zeros((1, K), np.uint16)
        x[0, j] = 0x3F80  # 1.0
        y, _ = oracle.spmv(m, v, x, K)
        assert (y[0] == pins.bf16_to_f64(Wp[:, j])).all()


def test_spmv_power_of_two_scaling():
    R, K = 16, 256
    W = synth.weights(R, K, 71)
    n = oracle.col_norm(synth.calib_acts(K, 71))
    m, v = oracle.prune_pack(W, n, 2, 4)
    x = synth.decode_x(1, K, 71)
    y1, _ = oracle.spmv(m, v, x, K)
    x4 = synth.to_bf16_bits(synth.bf16_bits_to_f32(x) * 4.0)
    y4, _ = oracle.spmv(m, v, x4, K)
    assert (y4 == 4.0 * y1).all()


def test_thread_count_does_not_change_bits():
    R, K = 50, 320
    W = synth.weights(R, K, 81)
    x = synth.decode_x(2, K, 81)
    y1, a1 = oracle.dense(W, x, nthreads=1)
    y7, a7 = oracle.dense(W, x, nthreads=7)
    assert (y1 == y7).all() and (a1 == a7).all()


# ------------------------------------------------------------------ error paths
def test_oracle_rejects_out_of_contract_inputs():
    W = synth.weights(4, 64, 1)
    n = np.ones(64, np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.prune_pack(W, n, 3, 4)  # not 50%
    with pytest.raises(oracle.OracleError):
        oracle.prune_pack(W, n, 1, 2)  # M not in {4,8,16,32}
    Wbad = W.copy()
    Wbad[1, 3] = 0x7FC0  # NaN
    with pytest.raises(oracle.OracleError):
        oracle.prune_pack(Wbad, n, 2, 4)
    m, v = oracle.prune_pack(W, n, 2, 4)
    mbad = m.copy()
    mbad[0, 0] = np.uint32(0x0001FFFF)  # 17 set bits
    with pytest.raises(oracle.OracleError):
        oracle.spmv(mbad, v, synth.decode_x(1, 64, 1), 64)
    with pytest.raises(oracle.OracleError):
        oracle.col_norm(np.full((2, 4), 0x7F80, np.uint16))  # +inf


# ------------------------------------------------------------------ mutation tests
# A plausible mistake planted in the oracle's output must trip a pin.
def test_mutant_ties_to_higher_index_is_caught():
    W, n = synth.tie_stress(16, 128, 91)
    m, _ = oracle.prune_pack(W, n, 2, 4)
    # mutant: among equal scores keep the higher column (reverse each group, re-run, reverse back)
    Wrev = W.reshape(16, 32, 4)[..., ::-1].reshape(16, 128).copy()
    nrev = n.reshape(32, 4)[:, ::-1].reshape(128).copy()
    mr, _ = oracle.prune_pack(Wrev, nrev, 2, 4)
    bits = pins.mask_bits(mr, 128).reshape(16, 32, 4)[..., ::-1].reshape(16, 128)
    mutant = pins.masks_from_bits(bits)
    assert (pins.mask_bits(mutant, 128) == bits).all()
    assert not (mutant == m).all()
    assert not pins.certificate_ok(W, n, mutant, 2, 4).all()


def test_mutant_msb_first_bit_order_is_caught():
    W, n, keep, mask, _, _ = _load_worked()
    Wb = synth.to_bf16_bits(W)[None, :]
    m, _ = oracle.prune_pack(Wb, n, 2, 4)
    mutant = int("{:032b}".format(int(m[0, 0]))[::-1], 2)  # bit b <-> column 31-b
    assert mutant != mask["2:4"]


def test_mutant_value_order_is_caught():
    W = synth.weights(8, 128, 93)
    n = oracle.col_norm(synth.calib_acts(128, 93))
    m, v = oracle.prune_pack(W, n, 4, 8)
    mutant = v.reshape(8, 4, 16)[..., ::-1].reshape(8, 64)  # descending inside each word
    assert not (pins.pack_by_indexing(W, m) == mutant).all()


def test_mutant_dropped_term_is_caught():
    R, K = 8, 128
    W = synth.weights(R, K, 94)
    n = oracle.col_norm(synth.calib_acts(K, 94))
    m, v = oracle.prune_pack(W, n, 2, 4)
    x = synth.decode_x(1, K, 94)
    y, _ = oracle.spmv(m, v, x, K)
    Wp = pins.bf16_to_f64(pins.unpack_by_indexing(m, v, K))
    xf = pins.bf16_to_f64(x)
    mutant = y.copy()
    last = np.nonzero(Wp[0])[0][-1]
    mutant[0, 0] -= Wp[0, last] * xf[0, last]  # forgot the last kept weight of row 0
    ref = xf @ Wp.T
    assert not np.allclose(mutant, ref, rtol=1e-12, atol=0)


def test_mutant_extra_kept_weight_is_caught():
    W = synth.weights(4, 64, 95)
    n = oracle.col_norm(synth.calib_acts(64, 95))
    m, _ = oracle.prune_pack(W, n, 2, 4)
    mutant = m.copy()
    free = [b for b in range(32) if not (int(mutant[0, 0]) >> b) & 1][0]
    mutant[0, 0] |= np.uint32(1 << free)
    assert not pins.certificate_ok(W, n, mutant, 2, 4).all()
    assert (pins.popcounts(mutant) != 16).any()


def test_tiny_regression_digests():
    """Regression only: digests written by tests/golden/make_golden.py from the oracle."""
    import hashlib
    import json

    from tests.golden.make_golden import N as GN, M as GM, K as GK, tiny_inputs

    with open(os.path.join(GOLDEN, "tiny_2of4_seed0.json")) as f:
        fx = json.load(f)
    W, X, x = tiny_inputs()
    h = lambda a: hashlib.sha256(a.tobytes()).hexdigest()  # noqa: E731
    assert h(W) == fx["sha256_W"] and h(X) == fx["sha256_X"] and h(x) == fx["sha256_x"]
    n = oracle.col_norm(X)
    m, v = oracle.prune_pack(W, n, GN, GM)
    y, _ = oracle.spmv(m, v, x, GK)
    assert h(n) == fx["sha256_col_norm"] and h(m) == fx["sha256_masks"] and h(v) == fx["sha256_values"]
    assert h(y) == fx["sha256_y_ref"]
