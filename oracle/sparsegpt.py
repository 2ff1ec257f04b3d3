"""CPU oracle of the OBS / SparseGPT N:M solver -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
use this module; it shares nothing with the HIP library.  Plain numpy in fp64; numpy's
matmul, Cholesky and inverse serve as library steps.

What it follows (pages cited by title and section):

* "SparseDecoding:解码感知的准确高效大模型剪枝框架" (paper.rainbus.top), 前置知识
  (训练后剪枝与OBS框架) and 方法步骤详情 第二步: the layer Hessian H = 2 X X^T of the
  calibration activations; the saliency of weight q is w_q^2 / (2 [H^-1]_qq); the weight
  with the smallest saliency is removed and the remaining weights are compensated by
  delta_w = -(w_q / [H^-1]_qq) H^-1_{:,q}; SparseGPT makes this feasible at scale and
  runs until the target pattern (50%, 2:4, ...) is reached.
* "SparseDecoding: Decoding-Aware Pruning ..." (ai.info summary), Methodology Step 1:
  the activations define a Hessian that decides which weights are removed and how the
  survivors are adjusted; the solver itself is unmodified.

Readings taken (the pages give the OBS formulas, not SparseGPT's schedule):

* SparseGPT's published column-sequential schedule: columns are processed left to
  right; once processed, a column is frozen, so the inverse Hessian that applies to
  column i is that of the columns not yet processed, (H_{i:,i:})^-1.  The upper
  Cholesky factor U of H^-1 (H^-1 = U^T U) carries all of them at once:
  U[i,i]^2 = [(H_{i:,i:})^-1]_ii and the OBS update of column i onto the columns after
  it is -(err_i) * U[i, i+1:] with err_i = (w_i - w_i_new) / U[i,i].
* N:M selection: at the first column of every group of M columns, each row keeps the N
  columns of the group with the largest saliency w^2 / U[c,c]^2 (current, already
  compensated weights; the factor 2 of the pages' saliency is common to all and does
  not change the order); ties keep the lower column, as in the Wanda selection.
* Damping: H + lambda I with lambda = damp * mean(diag H) (SparseGPT's dampening;
  damp = 0.01 by default).
* Output: the kept weights after compensation, rounded once to bf16 (nearest even),
  packed like any other N:M matrix (mask bits + values in increasing column order).
"""
from __future__ import annotations

import numpy as np


def _bf16_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _f64_to_bf16(v) -> np.ndarray:
    """Round fp64 once to the nearest bf16 (ties to even) -> bit patterns.  With
    v = m * 2^e, 1/2 <= |m| < 1, a normal bf16 keeps 8 significant bits:
    rint(m * 2^8) * 2^(e-8); below 2^-126 the spacing is fixed at 2^-133."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    normal = np.rint(m * 256.0) * np.exp2(e.astype(np.float64) - 8.0)
    sub = np.rint(v * 2.0 ** 133) * 2.0 ** -133
    r = np.where(np.abs(v) < 2.0 ** -126, sub, normal)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)  # exact: r has at most 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def hessian(X) -> np.ndarray:
    """H = 2 X^T X for calibration activations X: bf16 bit patterns [T][K] (tokens by input
    channels) -> fp64 [K][K].  Products of two bf16 values are exact in fp64."""
    Xf = _bf16_to_f64(X)
    return 2.0 * (Xf.T @ Xf)


def damped(H, damp: float) -> np.ndarray:
    H = np.array(H, dtype=np.float64, copy=True)
    lam = damp * float(np.mean(np.diag(H)))
    H[np.diag_indices_from(H)] += lam
    return H


def inverse_factor(H, damp: float) -> np.ndarray:
    """Upper-triangular U with positive diagonal and U^T U = (H + lambda I)^-1."""
    Hinv = np.linalg.inv(damped(H, damp))
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T  # numpy returns the lower factor L with L L^T


def _keep_group(sal_row, N: int) -> np.ndarray:
    """Indices (within the group) of the N kept columns: largest saliency first, ties to
    the lower column."""
    order = sorted(range(len(sal_row)), key=lambda c: (-sal_row[c], c))
    return np.array(sorted(order[:N]), dtype=np.int64)


def prune(W, H, N: int, M: int, damp: float = 0.01):
    """Column-sequential OBS with N:M selection.

    W: bf16 bit patterns [R][K]; H: fp64 [K][K].  Returns (keep bool [R][K], Wc fp64 [R][K]
    with the compensated weights, pruned entries 0)."""
    if not (M in (4, 8, 16, 32) and 2 * N == M):
        raise ValueError("50% N:M patterns with M in {4, 8, 16, 32} only")
    Wc = _bf16_to_f64(W).copy()
    R, K = Wc.shape
    if K % M:
        raise ValueError("K must be a multiple of M")
    U = inverse_factor(H, damp)
    d = np.diag(U)
    keep = np.zeros((R, K), dtype=bool)
    for i in range(K):
        if i % M == 0:
            sal = Wc[:, i:i + M] ** 2 / d[i:i + M] ** 2
            for r in range(R):
                keep[r, i + _keep_group(sal[r], N)] = True
        q = Wc[:, i].copy()
        new = np.where(keep[:, i], q, 0.0)
        err = (q - new) / d[i]
        Wc[:, i] = new
        Wc[:, i + 1:] -= np.outer(err, U[i, i + 1:])
    return keep, Wc


def prune_pack(W, H, N: int, M: int, damp: float = 0.01):
    """prune() followed by the bitmask packing -> (masks uint32 [R][K/32], values bf16 [R][K/2])."""
    keep, Wc = prune(W, H, N, M, damp)
    R, K = keep.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    bits = keep.reshape(R, K // 32, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)
    masks = bits.sum(axis=2).astype(np.uint32)
    values = _f64_to_bf16(Wc[keep]).reshape(R, K // 2)
    return masks, values


def reconstruction_error(W, Wc, X) -> np.ndarray:
    """Per row ||(W - Wc) X^T||^2 with X [T][K] (bf16 patterns) and W the original bf16."""
    Xf = _bf16_to_f64(X)
    D = _bf16_to_f64(W) - np.asarray(Wc, dtype=np.float64)
    return np.sum((D @ Xf.T) ** 2, axis=1)
