"""Pins for the OBS / SparseGPT solver oracle (oracle/sparsegpt.py).

Tied to things other than itself: exact rational Hessians, the defining property of
the inverse factor checked through independent inverses of every trailing submatrix,
the diagonal-Hessian special case (no compensation; the selection becomes Wanda's),
a from-scratch least-squares re-solve of the free columns after every fixed column
(an independent route to the whole compensation sequence), the objective never
exceeding the uncompensated one for the same mask, the N:M structure and the packing,
and planted mistakes.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import sparsegpt as sg
from tests import pins

PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]


def small_ints(shape, seed):
    """bf16 bit patterns of small integers in [-3, 3] (exact in every precision used)."""
    v = synth.rng(seed).integers(-3, 4, size=shape).astype(np.float32)
    return synth.to_bf16_bits(v)


def test_hessian_exact_rationals():
    X = small_ints((9, 6), 1)
    Xf = pins.bf16_to_f64(X)
    H = sg.hessian(X)
    for i in range(6):
        for j in range(6):
            exact = 2 * sum(Fraction(float(Xf[t, i])) * Fraction(float(Xf[t, j])) for t in range(9))
            assert H[i, j] == float(exact)


def test_hessian_bf16_products_exact_on_real_data():
    X = synth.calib_acts(40, 2, T=16)
    Xf = pins.bf16_to_f64(X)
    H = sg.hessian(X)
    ref = np.array([[2 * float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(Xf[:, i], Xf[:, j])))
                     for j in range(40)] for i in range(40)])
    assert np.allclose(H, ref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("damp", [0.01, 0.1])
def test_inverse_factor_properties(damp):
    X = synth.calib_acts(48, 3, T=32)
    H = sg.hessian(X)
    U = sg.inverse_factor(H, damp)
    Hd = sg.damped(H, damp)
    assert np.allclose(np.tril(U, -1), 0)
    assert (np.diag(U) > 0).all()
    assert np.allclose(U.T @ U @ Hd, np.eye(48), atol=1e-9)
    # U[i,i]^2 is the inverse Hessian entry of column i among the columns not yet processed
    for i in range(48):
        sub = np.linalg.inv(Hd[i:, i:])
        assert abs(U[i, i] ** 2 - sub[0, 0]) <= 1e-10 * sub[0, 0]


def test_damping_scale():
    H = np.diag([1.0, 3.0, 8.0])
    Hd = sg.damped(H, 0.5)
    assert np.allclose(np.diag(Hd), [1 + 2, 3 + 2, 8 + 2])


@pytest.mark.parametrize("N,M", PATTERNS)
def test_diagonal_hessian_is_wanda_without_compensation(N, M):
    """Orthogonal calibration columns: H is diagonal, the inverse factor has no
    off-diagonal entries, nothing is compensated, and the saliency w^2 * H_cc orders
    like Wanda's |w| * ||X_c|| -- the masks equal the Wanda oracle's."""
    R, K = 12, 64
    s = synth.rng(4, M).choice([0.5, 1.0, 2.0, 4.0, 0.25, 8.0], size=K).astype(np.float32)
    X = np.zeros((K, K), np.float32)
    X[np.arange(K), np.arange(K)] = s
    Xb = synth.to_bf16_bits(X)
    W = synth.weights(R, K, 5, M)
    H = sg.hessian(Xb)
    masks, values = sg.prune_pack(W, H, N, M, damp=0.0)
    mw, vw = oracle.prune_pack(W, oracle.col_norm(Xb), N, M)
    assert (masks == mw).all()
    assert (values == vw).all()


def _resolve_reference(W, H, N, M, damp):
    """Independent route: after fixing column i (kept value or 0), re-solve the free
    columns i+1.. from scratch by least squares against the damped Hessian."""
    Hd = sg.damped(H, damp)
    w0 = pins.bf16_to_f64(W)
    R, K = w0.shape
    cur = w0.copy()
    keep = np.zeros((R, K), dtype=bool)
    for i in range(K):
        if i % M == 0:
            dsq = np.array([np.linalg.inv(Hd[c:, c:])[0, 0] for c in range(i, i + M)])
            sal = cur[:, i:i + M] ** 2 / dsq
            for r in range(R):
                order = sorted(range(M), key=lambda c: (-sal[r, c], c))[:N]
                keep[r, [i + c for c in order]] = True
        cur[:, i] = np.where(keep[:, i], cur[:, i], 0.0)
        if i + 1 < K:
            A = Hd[i + 1:, i + 1:]
            Bm = Hd[i + 1:, :i + 1]
            # free z minimises (w0 - [fixed, z]) Hd (w0 - [fixed, z])^T
            cur[:, i + 1:] = w0[:, i + 1:] + np.linalg.solve(A, Bm @ (w0[:, :i + 1] - cur[:, :i + 1]).T).T
    return keep, cur


@pytest.mark.parametrize("N,M,K", [(2, 4, 16), (4, 8, 32), (8, 16, 32)])
def test_compensation_equals_least_squares_resolve(N, M, K):
    R = 6
    W = synth.weights(R, K, 6, K)
    X = synth.calib_acts(K, 6, K, T=2 * K)
    H = sg.hessian(X)
    keep, Wc = sg.prune(W, H, N, M, damp=0.01)
    kref, wref = _resolve_reference(W, H, N, M, 0.01)
    assert (keep == kref).all()
    assert np.allclose(Wc, wref, rtol=1e-8, atol=1e-12)


@pytest.mark.parametrize("N,M", PATTERNS)
def test_structure_packing_and_objective(N, M):
    R, K = 20, 128
    W = synth.weights(R, K, 7, M)
    X = synth.calib_acts(K, 7, M, T=64)
    H = sg.hessian(X)
    keep, Wc = sg.prune(W, H, N, M)
    assert (keep.reshape(R, K // M, M).sum(-1) == N).all()
    assert (Wc[~keep] == 0).all()
    masks, values = sg.prune_pack(W, H, N, M)
    assert (pins.mask_bits(masks, K) == keep).all()
    assert (pins.popcounts(masks) == 16).all()
    # values are the compensated kept weights, each rounded once to bf16
    back = pins.bf16_to_f64(oracle.unpack(masks, values, K))
    assert np.all(np.abs(back[keep] - Wc[keep]) <= 2.0 ** -8 * np.abs(Wc[keep]))
    # compensation never loses against the same mask left uncompensated
    plain = np.where(keep, pins.bf16_to_f64(W), 0.0)
    e_sgpt = sg.reconstruction_error(W, Wc, X)
    e_plain = sg.reconstruction_error(W, plain, X)
    assert (e_sgpt <= e_plain * (1 + 1e-9) + 1e-18).all()
    assert e_sgpt.sum() < e_plain.sum()


def test_bf16_rounding_definition():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, -0.0, 2.0 ** -130,
                  3 * 2.0 ** -134, 0.02, -1.5 - 2 ** -9])
    got = sg._f64_to_bf16(v)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x8000, 0x0008, 0x0002, 0x3CA4, 0xBFC0]
    # against the fp32 route on values that are exact in fp32 (no double rounding there)
    f = synth.rng(8).normal(0, 1, 1000).astype(np.float32).astype(np.float64)
    assert (sg._f64_to_bf16(f) == synth.to_bf16_bits(f.astype(np.float32))).all()


def test_mutant_without_compensation_is_caught():
    R, K, N, M = 6, 32, 4, 8
    W = synth.weights(R, K, 9)
    X = synth.calib_acts(K, 9, T=64)
    H = sg.hessian(X)
    keep, Wc = sg.prune(W, H, N, M)
    mutant = np.where(keep, pins.bf16_to_f64(W), 0.0)
    kref, wref = _resolve_reference(W, H, N, M, 0.01)
    assert not np.allclose(mutant, wref, rtol=1e-8, atol=1e-12)
    assert np.allclose(Wc, wref, rtol=1e-8, atol=1e-12)
