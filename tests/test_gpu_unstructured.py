"""GPU parity of the 50% unstructured path against the oracle: masks, packed values and
the unpacked matrix bit-exact; the SpMV within the same tolerance as the N:M kernel
(|y - y_ref| <= 1e-2 |y_ref| + 1e-3 sum_j |W_ij x_j|), exact on integer data."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import pins
from tests.gpu_util import bf16_as_f64, dev_bf16, dev_f32, dev_u32, host_bf16, host_u32, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402

RTOL, ATOL_FRAC = 1e-2, 1e-3


def assert_within(y_bits, y_ref, absum, what):
    y = bf16_as_f64(y_bits)
    ok = oracle.within_tolerance(y, y_ref, absum, RTOL, ATOL_FRAC)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside, e.g. {i}: {y[i]} vs {y_ref[i]}")


@pytest.mark.parametrize("R,K", [(64, 512), (37, 1024), (1, 32), (300, 4096), (8, 14336)])
def test_pack_and_unpack_bit_exact(R, K):
    say("unstructured pack", R, K)
    W = synth.weights(R, K, 21, R, K)
    X = synth.calib_acts(K, 21, R, K)
    n = nm.nm_col_norm(dev_bf16(X))
    m, v = nm.nm_prune_pack_unstructured(dev_bf16(W), n)
    U = nm.nm_unpack_unstructured(m, v)
    torch.cuda.synchronize()
    mref, vref = oracle.prune_pack_unstructured(W, oracle.col_norm(X))
    assert (host_u32(m) == mref).all()
    assert (host_bf16(v) == vref).all()
    assert (host_bf16(U) == oracle.unpack_unstructured(mref, vref, K)).all()


def test_pack_tie_stress_and_zero_norms():
    say("unstructured pack ties")
    W, n = synth.tie_stress(40, 1024, 22)
    n = n.copy()
    n[::7] = 0.0  # zero-norm columns: every score 0, ties broken by column
    m, v = nm.nm_prune_pack_unstructured(dev_bf16(W), dev_f32(n))
    torch.cuda.synchronize()
    mref, vref = oracle.prune_pack_unstructured(W, n)
    assert (host_u32(m) == mref).all()
    assert (host_bf16(v) == vref).all()


SHAPES = [(256, 512), (1000, 4096), (513, 5120), (96, 14336), (17, 8192), (3, 28672), (1, 32)]


@pytest.mark.parametrize("R,K", SHAPES)
@pytest.mark.parametrize("B", [1, 3, 8])
def test_spmv_within_tolerance(R, K, B):
    say("unstructured spmv", R, K, B)
    W = synth.weights(R, K, 23, R, K)
    mref, vref = oracle.prune_pack_unstructured(W, oracle.col_norm(synth.calib_acts(K, 23, R, K)))
    x = synth.decode_x(B, K, 23, R, K, B)
    y = nm.nm_spmv_unstructured(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    y2 = nm.nm_spmv_unstructured(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    torch.cuda.synchronize()
    yref, absum = oracle.spmv_unstructured(mref, vref, x, K, nthreads=4)
    assert_within(host_bf16(y), yref, absum, f"R={R} K={K} B={B}")
    assert (host_bf16(y) == host_bf16(y2)).all()


def test_spmv_integer_exact_and_skewed_words():
    """Ternary data with a column norm that concentrates the kept weights in a few words
    (full and empty words side by side): results are exact integers."""
    say("unstructured integer")
    R, K, B = 64, 2048, 2
    W = synth.ternary((R, K), 24)
    W[:, :64] = synth.to_bf16_bits(np.ones((R, 64), np.float32))  # two words fully kept
    n = np.ones(K, np.float32)
    n[: K // 2] = 4.0  # favour the first half: many words fully kept, many empty
    mref, vref = oracle.prune_pack_unstructured(W, n)
    pc = pins.popcounts(mref)
    assert pc.max() == 32 and pc.min() == 0
    x = synth.ternary((B, K), 25)
    y = nm.nm_spmv_unstructured(dev_u32(mref), dev_bf16(vref), dev_bf16(x))
    torch.cuda.synchronize()
    yref, _ = oracle.spmv_unstructured(mref, vref, x, K)
    assert (bf16_as_f64(host_bf16(y)) == yref).all()


def test_full_size_sampled():
    """Llama-3.1-8B gate shape (14336 x 4096), generated and packed on the device."""
    R, K, B = 14336, 4096, 1
    say("unstructured full", R, K)
    Wd = synth.device_weights(R, K, 5, R, K)
    Xd = synth.device_calib_acts(K, 5, K)
    xd = synth.device_decode_x(B, K, 5, K, B)
    n = nm.nm_col_norm(Xd)
    m, v = nm.nm_prune_pack_unstructured(Wd, n)
    y = nm.nm_spmv_unstructured(m, v, xd)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, R - 1], np.random.default_rng(9).choice(R, 160, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    Ws = host_bf16(Wd.index_select(0, ridx))
    ms, vs = oracle.prune_pack_unstructured(Ws, oracle.col_norm(host_bf16(Xd)))
    assert (host_u32(m.index_select(0, ridx)) == ms).all()
    assert (host_bf16(v.index_select(0, ridx)) == vs).all()
    yref, absum = oracle.spmv_unstructured(ms, vs, host_bf16(xd), K, nthreads=4)
    assert_within(host_bf16(y)[:, rows], yref, absum, "8b gate unstructured")
