"""GPU parity of the index-metadata path (uint8 offsets, int32 column indices): the
conversion kernel bit-exact against the oracle, and the SpMV over each format within
the SpMV tolerance of the oracle's direct index-metadata matvec.  The uint8 path walks
each word in the same lane and order as the word-per-lane bitmask kernel, so where
nm_spmv takes that kernel its outputs are also bit-identical to nm_spmv's (where
nm_spmv takes the matrix-core tile kernel, the fp32 summation order differs and both
are held to the tolerance); the int32 path spreads a word over four lanes (another fp32
summation order), so it is held to the tolerance and to run-to-run determinism."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_as_f64, dev_bf16, dev_u32, host_bf16, host_u32, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402

RTOL, ATOL_FRAC = 1e-2, 1e-3
FMTS = [(nm.NM_META_U8_OFFSET, oracle.META_U8), (nm.NM_META_I32_INDEX, oracle.META_I32)]


def _host_meta(t: torch.Tensor) -> np.ndarray:
    a = t.contiguous().cpu().numpy()
    return a.view(np.uint8) if a.dtype == np.uint8 else a.view(np.int32)


def _pack(R, K, M, *ids):
    W = synth.weights(R, K, 17, *ids)
    return oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 17, *ids)), M // 2, M)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("R,K,M", [(64, 512, 4), (37, 1024, 32), (1, 32, 8), (300, 4096, 16)])
def test_meta_from_mask_bit_exact(fmt, ofmt, R, K, M):
    say("meta_from_mask", fmt, R, K, M)
    m, _ = _pack(R, K, M, R, K)
    got = _host_meta(nm.nm_meta_from_mask(dev_u32(m), fmt))
    ref = oracle.meta_from_mask(m, K, ofmt)
    assert got.shape == ref.shape and (got == ref).all()


SHAPES = [(256, 512), (129, 4096), (1000, 1024), (7, 14336), (1, 32), (3, 28672)]


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("R,K", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 3, 8])
def test_spmv_meta_matches_oracle_and_bitmask(fmt, ofmt, R, K, B):
    say("spmv_meta", fmt, R, K, B)
    m, v = _pack(R, K, 8, R, K, B)
    meta = oracle.meta_from_mask(m, K, ofmt)
    x = synth.decode_x(B, K, 17, R, K, B)
    xd, vd = dev_bf16(x), dev_bf16(v)
    meta_d = torch.from_numpy(np.ascontiguousarray(meta)).cuda()
    y = nm.nm_spmv_meta(meta_d, fmt, vd, xd)
    y2 = nm.nm_spmv_meta(meta_d, fmt, vd, xd)
    yb = nm.nm_spmv(dev_u32(m), vd, xd)
    torch.cuda.synchronize()
    yref, absum = oracle.spmv_index(meta, ofmt, v, x, K, nthreads=4)
    got = bf16_as_f64(host_bf16(y))
    ok = oracle.within_tolerance(got, yref, absum, RTOL, ATOL_FRAC)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outside tolerance"
    assert (host_bf16(y) == host_bf16(y2)).all()
    if fmt == nm.NM_META_U8_OFFSET and nm.nm_spmv_plan(R, K, B)["kernel"] == nm.NM_KERNEL_WORD:
        assert (host_bf16(y) == host_bf16(yb)).all()
    else:
        okb = oracle.within_tolerance(bf16_as_f64(host_bf16(yb)), yref, absum, RTOL, ATOL_FRAC)
        assert okb.all(), f"nm_spmv: {int((~okb).sum())} of {okb.size} outside tolerance"


def test_spmv_meta_bitmask_format_is_nm_spmv():
    say("spmv_meta bitmask")
    R, K, B = 500, 2048, 2
    m, v = _pack(R, K, 4, 99)
    x = dev_bf16(synth.decode_x(B, K, 99))
    md = dev_u32(m)
    y0 = nm.nm_spmv_meta(md, nm.NM_META_BITMASK, dev_bf16(v), x)
    y1 = nm.nm_spmv(md, dev_bf16(v), x)
    torch.cuda.synchronize()
    assert (host_bf16(y0) == host_bf16(y1)).all()


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_spmv_meta_full_size_sampled(fmt, ofmt):
    """8B MLP up-projection shape (14336 x 4096), packed and converted on the device."""
    R, K, B = 14336, 4096, 1
    say("spmv_meta full", fmt, R, K)
    Wd = synth.device_weights(R, K, 3, R, K)
    Xd = synth.device_calib_acts(K, 3, K)
    xd = synth.device_decode_x(B, K, 3, K, B)
    masks, values = nm.nm_prune_pack(Wd, nm.nm_col_norm(Xd), 2, 4)
    meta = nm.nm_meta_from_mask(masks, fmt)
    y = nm.nm_spmv_meta(meta, fmt, values, xd)
    yb = nm.nm_spmv(masks, values, xd)
    torch.cuda.synchronize()
    if fmt == nm.NM_META_U8_OFFSET:
        assert (host_bf16(y) == host_bf16(yb)).all()
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, R - 1], g.choice(R, size=128, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    ms = host_u32(masks.index_select(0, ridx))
    vs = host_bf16(values.index_select(0, ridx))
    meta_s = _host_meta(meta.index_select(0, ridx))
    assert (meta_s == oracle.meta_from_mask(ms, K, ofmt)).all()
    yref, absum = oracle.spmv_index(meta_s, ofmt, vs, host_bf16(xd), K, nthreads=4)
    got = bf16_as_f64(host_bf16(y)[:, rows])
    assert oracle.within_tolerance(got, yref, absum, RTOL, ATOL_FRAC).all()


def test_index_entries_are_confined_to_their_word():
    """An index that breaks the 50% N:M rule reads a column of its own word (low five
    bits), never memory outside x: the result equals the oracle on the reduced entries."""
    say("spmv_meta reduced entries")
    R, K = 32, 256
    m, v = _pack(R, K, 4, 7)
    idx = oracle.meta_from_mask(m, K, oracle.META_I32)
    bad = idx.copy()
    bad[:, 0] += 32 * 1000  # far outside the row
    x = synth.decode_x(1, K, 7)
    y = nm.nm_spmv_meta(torch.from_numpy(bad).cuda(), nm.NM_META_I32_INDEX, dev_bf16(v), dev_bf16(x))
    yok = nm.nm_spmv_meta(torch.from_numpy(idx).cuda(), nm.NM_META_I32_INDEX, dev_bf16(v), dev_bf16(x))
    torch.cuda.synchronize()
    assert (host_bf16(y) == host_bf16(yok)).all()
