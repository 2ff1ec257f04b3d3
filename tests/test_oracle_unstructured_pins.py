"""Pins for the oracle's 50% unstructured functions (prune_pack_unstructured,
unpack_unstructured, spmv_unstructured).

The pages' other 50% setting ("SparseDecoding: Decoding-Aware Pruning ...",
Methodology Step 4) keeps half of the weights without the N:M group constraint; the
reading taken is Wanda's unstructured rule: each row keeps its K/2 highest scores
(ties to the lower column), encoded with the same bitmask and ascending values.
Pinned by a per-row certificate, the 16:32 pack (one group = the whole row at K = 32)
and the hand-worked row, brute force with exact rationals on restricted rows, numpy
boolean-index unpack and fp64 matmul, integer sums, and planted mistakes.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import pins
from tests.test_oracle_pins import _load_worked


def row_certificate(W, n, masks) -> np.ndarray:
    """Per row: exactly K/2 kept, and every kept (score, col) precedes every dropped one
    under (score desc, col asc)."""
    R, K = W.shape
    kept = pins.mask_bits(masks, K)
    s = pins.exact_scores(W, n)
    col = np.broadcast_to(np.arange(K)[None, :], kept.shape)
    count_ok = kept.sum(1) == K // 2
    ks = np.where(kept, s, np.inf).min(1)
    ds = np.where(~kept, s, -np.inf).max(1)
    kc = np.where(kept & (s == ks[:, None]), col, -1).max(1)
    dc = np.where(~kept & (s == ds[:, None]), col, np.iinfo(np.int64).max).min(1)
    return count_ok & ((ks > ds) | ((ks == ds) & (kc < dc)))


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("K", [32, 256, 1024])
def test_certificate_random(seed, K):
    R = 40
    W = synth.weights(R, K, seed, K)
    n = oracle.col_norm(synth.calib_acts(K, seed, K))
    m, _ = oracle.prune_pack_unstructured(W, n)
    assert row_certificate(W, n, m).all()


def test_certificate_tie_stress():
    W, n = synth.tie_stress(24, 512, 3)
    m, _ = oracle.prune_pack_unstructured(W, n)
    assert row_certificate(W, n, m).all()


def test_word_popcounts_vary_but_rows_hold_half():
    R, K = 64, 1024
    W = synth.weights(R, K, 4)
    n = oracle.col_norm(synth.calib_acts(K, 4))
    m, _ = oracle.prune_pack_unstructured(W, n)
    pc = pins.popcounts(m)
    assert (pc.sum(1) == K // 2).all()
    assert pc.min() < 16 < pc.max()  # not an N:M pattern


def test_whole_row_group_equals_16_of_32():
    """At K = 32 a row is one 32-column group: unstructured == 16:32."""
    W = synth.weights(50, 32, 5)
    n = oracle.col_norm(synth.calib_acts(32, 5))
    mu, vu = oracle.prune_pack_unstructured(W, n)
    mn, vn = oracle.prune_pack(W, n, 16, 32)
    assert (mu == mn).all() and (vu == vn).all()


def test_worked_row_by_hand():
    W, n, keep, mask, _, _ = _load_worked()
    Wb = synth.to_bf16_bits(W)[None, :]
    m, v = oracle.prune_pack_unstructured(Wb, n)
    assert int(m[0, 0]) == mask["16:32"]
    assert [int(t) for t in v[0]] == [int(Wb[0, c]) for c in keep["16:32"]]


@pytest.mark.parametrize("K,live", [(32, 19), (64, 34)])
def test_brute_force_restricted_rows(K, live):
    """Rows where only `live` columns (> K/2) carry nonzero scores: the kept set is the
    best K/2-subset of the live columns -- maximal exact sum of scores, then the
    lexicographically smallest columns -- found by enumerating every subset."""
    g = synth.rng(6, K)
    for trial in range(10):
        W = np.zeros((1, K), np.float32)
        cols = np.sort(g.choice(K, live, replace=False))
        vals = g.choice([0.25, 0.5, 1.0, 2.0, -1.0, -0.5, 0.75], size=live)  # many ties
        W[0, cols] = vals
        Wb = synth.to_bf16_bits(W)
        n = np.ones(K, np.float32)
        m, _ = oracle.prune_pack_unstructured(Wb, n)
        kept = np.nonzero(pins.mask_bits(m, K)[0])[0].tolist()
        best = pins.brute_force_group(np.abs(vals), K // 2)
        assert kept == [int(cols[i]) for i in best]


@pytest.mark.parametrize("K", [64, 512])
def test_roundtrip_and_numpy_unpack(K):
    R = 30
    W = synth.weights(R, K, 7, K)
    n = oracle.col_norm(synth.calib_acts(K, 7, K))
    m, v = oracle.prune_pack_unstructured(W, n)
    U = oracle.unpack_unstructured(m, v, K)
    assert (U == pins.unpack_by_indexing(m, v, K)).all()
    assert (U == np.where(pins.mask_bits(m, K), W, 0)).all()


@pytest.mark.parametrize("B", [1, 4])
def test_spmv_vs_numpy_matmul(B):
    R, K = 48, 640
    W = synth.weights(R, K, 8, B)
    n = oracle.col_norm(synth.calib_acts(K, 8, B))
    m, v = oracle.prune_pack_unstructured(W, n)
    x = synth.decode_x(B, K, 8)
    y, a = oracle.spmv_unstructured(m, v, x, K, nthreads=2)
    Wp = pins.bf16_to_f64(pins.unpack_by_indexing(m, v, K))
    xf = pins.bf16_to_f64(x)
    assert np.allclose(y, xf @ Wp.T, rtol=1e-12, atol=1e-12 * a.max())
    assert np.allclose(a, np.abs(xf) @ np.abs(Wp).T, rtol=1e-12)


def test_spmv_integer_exact():
    R, K, B = 12, 256, 2
    W = synth.ternary((R, K), 9)
    x = synth.ternary((B, K), 10)
    n = oracle.col_norm(synth.calib_acts(K, 11))
    m, v = oracle.prune_pack_unstructured(W, n)
    wi = pins.bf16_to_f64(pins.unpack_by_indexing(m, v, K)).astype(np.int64)
    xi = pins.bf16_to_f64(x).astype(np.int64)
    y, _ = oracle.spmv_unstructured(m, v, x, K)
    assert (y == (xi @ wi.T).astype(np.float64)).all()


def test_rejects_rows_without_half_kept():
    R, K = 4, 64
    W = synth.weights(R, K, 12)
    n = oracle.col_norm(synth.calib_acts(K, 12))
    m, v = oracle.prune_pack_unstructured(W, n)
    bad = m.copy()
    bad[1, 0] ^= np.uint32(1 << (int(np.nonzero(pins.mask_bits(m, K)[1])[0][0]) % 32))  # drop one kept bit
    with pytest.raises(oracle.OracleError):
        oracle.spmv_unstructured(bad, v, synth.decode_x(1, K, 12), K)
    with pytest.raises(oracle.OracleError):
        oracle.unpack_unstructured(bad, v, K)


def test_mutant_nm_instead_of_rowwise_is_caught():
    """Planting the 8:16 pack in place of the row-wise one breaks the row certificate."""
    R, K = 16, 512
    W = synth.weights(R, K, 13)
    n = oracle.col_norm(synth.calib_acts(K, 13))
    mutant, _ = oracle.prune_pack(W, n, 8, 16)
    assert not row_certificate(W, n, mutant).all()
