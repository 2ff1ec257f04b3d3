"""Pins for the oracle's index-metadata functions (meta_from_mask, spmv_index).

The formats are the ones the bitmask is priced against on the pages
("SparseDecoding: Decoding-Aware Pruning ...", Main Findings, metadata reduction;
"SparseDecoding:解码感知的准确高效大模型剪枝框架", 核心方法 核心创新二): a uint8 offset
and an int32 column index per kept weight.  Pinned by the hand-worked fixture's kept
columns, the pages' bits-per-weight figures, a numpy scatter + matmul, integer sums,
and rejection of malformed metadata.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synth
from tests import pins
from tests.test_oracle_pins import _load_worked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]


def _metadata_fixture():
    fx = {}
    with open(os.path.join(GOLDEN, "metadata_bits.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                fx[k] = int(v)
    return fx


def test_worked_example_offsets_and_indices():
    """Two words: the 2:4 word, then the 4:8 word of the hand-worked row.  Offsets are the
    hand-listed kept columns of each word; indices add 32 for the second word."""
    _, _, keep, mask, _, _ = _load_worked()
    masks = np.array([[mask["2:4"], mask["4:8"]]], dtype=np.uint32)
    u8 = oracle.meta_from_mask(masks, 64, oracle.META_U8)
    i32 = oracle.meta_from_mask(masks, 64, oracle.META_I32)
    assert u8[0].tolist() == keep["2:4"] + keep["4:8"]
    assert i32[0].tolist() == keep["2:4"] + [32 + c for c in keep["4:8"]]


def test_bits_per_kept_weight_match_the_pages():
    fx = _metadata_fixture()
    R, K = 24, 512
    W = synth.weights(R, K, 3)
    n = oracle.col_norm(synth.calib_acts(K, 3))
    m, _ = oracle.prune_pack(W, n, 8, 16)
    nnz = R * K // 2
    u8 = oracle.meta_from_mask(m, K, oracle.META_U8)
    i32 = oracle.meta_from_mask(m, K, oracle.META_I32)
    assert u8.nbytes * 8 == fx["uint8_offset_bits_per_nnz"] * nnz
    assert i32.nbytes * 8 == fx["int32_index_bits_per_nnz"] * nnz
    assert i32.nbytes // m.nbytes == fx["ratio_vs_int32"]
    assert u8.nbytes // m.nbytes == fx["ratio_vs_uint8"]


@pytest.mark.parametrize("N,M", PATTERNS)
def test_metadata_lists_the_set_bits(N, M):
    """numpy route: column indices of the set bits, row by row (np.nonzero)."""
    R, K = 20, 320
    W = synth.weights(R, K, 5, M)
    n = oracle.col_norm(synth.calib_acts(K, 5, M))
    m, _ = oracle.prune_pack(W, n, N, M)
    bits = pins.mask_bits(m, K)
    cols = np.stack([np.nonzero(bits[i])[0] for i in range(R)])
    assert (oracle.meta_from_mask(m, K, oracle.META_I32) == cols).all()
    assert (oracle.meta_from_mask(m, K, oracle.META_U8) == cols % 32).all()


def _dense_from_index(idx, values, K):
    R = values.shape[0]
    Wd = np.zeros((R, K), np.float64)
    np.put_along_axis(Wd, idx.astype(np.int64), pins.bf16_to_f64(values), axis=1)
    return Wd


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("fmt", [oracle.META_U8, oracle.META_I32])
def test_spmv_index_vs_numpy_scatter_matmul(fmt, B):
    R, K = 72, 384
    W = synth.weights(R, K, 11, B)
    n = oracle.col_norm(synth.calib_acts(K, 11, B))
    m, v = oracle.prune_pack(W, n, 2, 4)
    meta = oracle.meta_from_mask(m, K, fmt)
    idx = meta.astype(np.int64)
    if fmt == oracle.META_U8:
        idx = idx + 32 * (np.arange(K // 2) // 16)[None, :]
    x = synth.decode_x(B, K, 11)
    y, a = oracle.spmv_index(meta, fmt, v, x, K, nthreads=2)
    Wd = _dense_from_index(idx, v, K)
    xf = pins.bf16_to_f64(x)
    ref = xf @ Wd.T
    aref = np.abs(xf) @ np.abs(Wd).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * aref.max())
    assert np.allclose(a, aref, rtol=1e-12)
    # and the bitmask oracle on the same weights sums the same products in the same order
    yb, ab = oracle.spmv(m, v, x, K)
    assert (y == yb).all() and (a == ab).all()


def test_spmv_index_integer_exact():
    R, K, B = 16, 256, 2
    W = synth.ternary((R, K), 21)
    x = synth.ternary((B, K), 22)
    n = oracle.col_norm(synth.calib_acts(K, 23))
    m, v = oracle.prune_pack(W, n, 16, 32)
    idx = oracle.meta_from_mask(m, K, oracle.META_I32)
    y, _ = oracle.spmv_index(idx, oracle.META_I32, v, x, K)
    vi = pins.bf16_to_f64(v).astype(np.int64)
    xi = pins.bf16_to_f64(x).astype(np.int64)
    for b in range(B):
        for i in range(R):
            assert y[b, i] == sum(int(vi[i, t]) * int(xi[b, idx[i, t]]) for t in range(K // 2))


def test_malformed_metadata_is_rejected():
    R, K = 4, 64
    W = synth.weights(R, K, 31)
    n = oracle.col_norm(synth.calib_acts(K, 31))
    m, v = oracle.prune_pack(W, n, 2, 4)
    x = synth.decode_x(1, K, 31)
    i32 = oracle.meta_from_mask(m, K, oracle.META_I32)
    u8 = oracle.meta_from_mask(m, K, oracle.META_U8)
    bad = i32.copy()
    bad[0, 16] = 5  # second word's first weight placed in the first word
    with pytest.raises(oracle.OracleError):
        oracle.spmv_index(bad, oracle.META_I32, v, x, K)
    bad = u8.copy()
    bad[1, 3], bad[1, 4] = bad[1, 4], bad[1, 3]  # not increasing
    with pytest.raises(oracle.OracleError):
        oracle.spmv_index(bad, oracle.META_U8, v, x, K)
    bad = u8.copy()
    bad[2, 15] = 32  # outside the word
    with pytest.raises(oracle.OracleError):
        oracle.spmv_index(bad, oracle.META_U8, v, x, K)
    mbad = m.copy()
    mbad[3, 1] = np.uint32(0x7FFF)  # 15 set bits
    with pytest.raises(oracle.OracleError):
        oracle.meta_from_mask(mbad, K, oracle.META_U8)


def test_mutant_missing_word_base_is_caught():
    """A plausible slip -- int32 indices without the 32w word base -- fails the numpy pin."""
    R, K = 8, 128
    W = synth.weights(R, K, 41)
    n = oracle.col_norm(synth.calib_acts(K, 41))
    m, v = oracle.prune_pack(W, n, 4, 8)
    good = oracle.meta_from_mask(m, K, oracle.META_I32)
    mutant = good % 32
    cols = np.stack([np.nonzero(pins.mask_bits(m, K)[i])[0] for i in range(R)])
    assert (good == cols).all()
    assert not (mutant == cols).all()
