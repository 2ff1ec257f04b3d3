"""GPU parity of the OBS / SparseGPT solver against the fp64 oracle (oracle/sparsegpt.py).

Both sides work in fp64, so the GPU may differ from the oracle only by summation order
(Hessian, Cholesky, triangular inverse, lazy block updates): H within 1e-12 relative,
the inverse factor within 1e-8 of its scale, masks identical, the packed bf16 values
identical except where the fp64 value lies within 1e-9 of a bf16 rounding boundary
(checked: such positions may differ by one bf16 step), and the reconstruction error
identical to 1e-6.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import sparsegpt as sg
from tests import pins
from tests.gpu_util import dev_bf16, host_bf16, host_u32, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402

PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]


@pytest.mark.parametrize("T,K", [(16, 32), (37, 64), (100, 100), (300, 512), (64, 4096)])
def test_hessian_matches_oracle(T, K):
    say("hessian", T, K)
    X = synth.calib_acts(K, 30, T, K, T=T)
    H = nm.nm_hessian(dev_bf16(X)).cpu().numpy()
    ref = sg.hessian(X)
    scale = np.sqrt(np.outer(np.diag(ref), np.diag(ref))) + 1e-300
    assert np.all(np.abs(H - ref) <= 1e-12 * scale)


@pytest.mark.parametrize("K", [32, 64, 256, 1024])
def test_inverse_factor_matches_oracle(K):
    say("inverse factor", K)
    X = synth.calib_acts(K, 31, K, T=max(16, K // 4))
    H = sg.hessian(X)
    Hd = torch.from_numpy(H).cuda()
    U = nm.nm_obs_inverse_factor(Hd, 0.01).cpu().numpy()
    Uref = sg.inverse_factor(H, 0.01)
    assert (np.tril(U, -1) == 0).all()
    assert np.max(np.abs(U - Uref)) <= 1e-8 * np.max(np.abs(Uref))
    assert np.allclose(U.T @ U @ sg.damped(H, 0.01), np.eye(K), atol=1e-6)


def _check_values(values_gpu, masks, W, H, N, M, damp):
    keep, Wc = sg.prune(W, H, N, M, damp)
    mref, vref = sg.prune_pack(W, H, N, M, damp)
    assert (masks == mref).all()
    diff = values_gpu != vref
    if diff.any():
        # allowed only next to a rounding boundary, and by one bf16 step
        kept = Wc[keep].reshape(vref.shape)
        lo = np.minimum(values_gpu, vref).astype(np.int64)
        hi = np.maximum(values_gpu, vref).astype(np.int64)
        assert np.all((hi - lo)[diff] == 1)
        mid = (pins.bf16_to_f64(vref[diff]) + pins.bf16_to_f64(values_gpu[diff])) / 2
        assert np.all(np.abs(kept[diff] - mid) <= 1e-9 * np.abs(kept[diff]))
    return mref, vref


@pytest.mark.parametrize("N,M", PATTERNS)
@pytest.mark.parametrize("R,K", [(64, 64), (100, 256), (33, 512)])
def test_prune_pack_matches_oracle(N, M, R, K):
    say("sparsegpt", N, M, R, K)
    W = synth.weights(R, K, 32, R, K, M)
    X = synth.calib_acts(K, 32, K, M, T=max(32, K // 2))
    H = sg.hessian(X)
    m, v = nm.nm_sparsegpt_prune_pack(dev_bf16(W), torch.from_numpy(H).cuda(), N, M, 0.01)
    torch.cuda.synchronize()
    masks, values = host_u32(m), host_bf16(v)
    assert (pins.popcounts(masks) == 16).all()
    _check_values(values, masks, W, H, N, M, 0.01)
    # reconstruction error of the packed result
    Wp = pins.bf16_to_f64(oracle.unpack(masks, values, K))
    mref, vref = sg.prune_pack(W, H, N, M, 0.01)
    Wr = pins.bf16_to_f64(oracle.unpack(mref, vref, K))
    e_gpu = sg.reconstruction_error(W, Wp, X)
    e_ref = sg.reconstruction_error(W, Wr, X)
    assert np.allclose(e_gpu, e_ref, rtol=1e-6, atol=0)


def test_gpu_hessian_feeds_the_solver():
    """End to end on the device: calibration X -> nm_hessian -> nm_sparsegpt_prune_pack,
    against the oracle run on the same X."""
    say("sparsegpt end to end")
    R, K, N, M = 48, 256, 2, 4
    W = synth.weights(R, K, 33)
    X = synth.calib_acts(K, 33, T=128)
    Hd = nm.nm_hessian(dev_bf16(X))
    m, v = nm.nm_sparsegpt_prune_pack(dev_bf16(W), Hd, N, M, 0.01)
    torch.cuda.synchronize()
    _check_values(host_bf16(v), host_u32(m), W, sg.hessian(X), N, M, 0.01)


def test_full_size_sampled_rows():
    """Llama-3.1-8B gate shape (14336 x 4096, 2:4) with 256 calibration tokens; rows are
    independent given H, so the oracle solves a sample of them."""
    R, K, N, M, T = 14336, 4096, 2, 4, 256
    say("sparsegpt full", R, K)
    Wd = synth.device_weights(R, K, 34, R, K)
    Xd = synth.device_calib_acts(K, 34, K, T=T)
    Hd = nm.nm_hessian(Xd)
    m, v = nm.nm_sparsegpt_prune_pack(Wd, Hd, N, M, 0.01)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, R - 1], np.random.default_rng(34).choice(R, 30, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    Ws = host_bf16(Wd.index_select(0, ridx))
    H = sg.hessian(host_bf16(Xd))
    assert np.all(np.abs(Hd.cpu().numpy() - H) <= 1e-12 * np.sqrt(np.outer(np.diag(H), np.diag(H))))
    _check_values(host_bf16(v.index_select(0, ridx)), host_u32(m.index_select(0, ridx)), Ws, H, N, M, 0.01)
