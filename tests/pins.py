"""Independent checkers used to pin the oracle (and, in the GPU tests, the HIP path).

None of these restates the oracle's code: the selection is checked through a
certificate (every kept score beats every dropped score of its group under the
tie rule) and through brute-force subset enumeration with exact rationals; the
packing through numpy boolean indexing; the matvec through numpy's fp64 matmul.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

import synth


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def mask_bits(masks: np.ndarray, K: int) -> np.ndarray:
    """uint32 [R, K/32] -> bool [R, K] with bit b of word w <-> column 32w+b."""
    masks = np.asarray(masks, dtype=np.uint32)
    R = masks.shape[0]
    shifts = np.arange(32, dtype=np.uint32)
    bits = (masks[:, :, None] >> shifts[None, None, :]) & np.uint32(1)
    return bits.reshape(R, K).astype(bool)


def exact_scores(W: np.ndarray, n: np.ndarray) -> np.ndarray:
    """|W| * n in fp64; exact because the significands are 8 and 24 bits wide."""
    return np.abs(bf16_to_f64(W)) * np.asarray(n, dtype=np.float32).astype(np.float64)[None, :]


def certificate_ok(W, n, masks, N: int, M: int) -> np.ndarray:
    """Per-group verdict (bool [R, K/M]): exactly N kept, and every kept (score, col)
    precedes every dropped one under (score desc, col asc)."""
    W = np.asarray(W)
    R, K = W.shape
    kept = mask_bits(masks, K).reshape(R, K // M, M)
    s = exact_scores(W, n).reshape(R, K // M, M)
    col = np.broadcast_to(np.arange(K).reshape(1, K // M, M), kept.shape)
    count_ok = kept.sum(-1) == N
    ks = np.where(kept, s, np.inf).min(-1)
    ds = np.where(~kept, s, -np.inf).max(-1)
    kc = np.where(kept & (s == ks[..., None]), col, -1).max(-1)
    dc = np.where(~kept & (s == ds[..., None]), col, np.iinfo(np.int64).max).min(-1)
    order_ok = (ks > ds) | ((ks == ds) & (kc < dc))
    return count_ok & order_ok


def pack_by_indexing(W, masks) -> np.ndarray:
    """Kept values in increasing column order, via numpy boolean indexing."""
    W = np.asarray(W, dtype=np.uint16)
    R, K = W.shape
    bits = mask_bits(masks, K)
    if not (bits.sum(1) == K // 2).all():
        raise AssertionError("a row does not keep exactly K/2 columns")
    return W[bits].reshape(R, K // 2)


def unpack_by_indexing(masks, values, K: int) -> np.ndarray:
    masks = np.asarray(masks, dtype=np.uint32)
    R = masks.shape[0]
    bits = mask_bits(masks, K)
    out = np.zeros((R, K), dtype=np.uint16)
    out[bits] = np.asarray(values, dtype=np.uint16).reshape(-1)
    return out


def brute_force_group(scores_row, N: int):
    """Keep-set maximising the exact sum of scores; among equal sums the
    lexicographically smallest index tuple (itertools yields tuples in that order)."""
    fr = [Fraction(float(v)) for v in scores_row]
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(fr)), N):
        t = sum((fr[i] for i in comb), Fraction(0))
        if best_sum is None or t > best_sum:
            best, best_sum = comb, t
    return best


def popcounts(masks) -> np.ndarray:
    m = np.asarray(masks, dtype=np.uint32)
    return np.unpackbits(m.view(np.uint8)).reshape(*m.shape, 32).sum(-1)


def rn64_sqrt(S: Fraction) -> float:
    """IEEE round-to-nearest fp64 value of the exact square root of a rational S >= 0
    (integer square root on a fine grid plus a sticky half-step)."""
    if S == 0:
        return 0.0
    k = 0
    while S * Fraction(4) ** k < Fraction(2) ** 160:
        k += 1
    scaled = S * Fraction(4) ** k
    N0 = scaled.numerator // scaled.denominator
    import math

    r = math.isqrt(N0)
    if r * r == scaled:  # exact square
        return float(Fraction(r, 2 ** k))
    # sqrt(S) lies strictly inside (r, r+1) / 2^k; with r >= 2^80 the interval is far
    # narrower than one fp64 ulp, and its midpoint rounds like sqrt(S) itself.
    return float(Fraction(2 * r + 1, 2 ** (k + 1)))


def exact_col_norm(X: np.ndarray) -> np.ndarray:
    """float32 [K]: fp32(RN64(sqrt(exact sum_t X[t][j]^2))) with the sum in exact rationals."""
    Xf = synth.bf16_bits_to_f32(np.asarray(X, dtype=np.uint16))
    T, K = Xf.shape
    out = np.empty(K, dtype=np.float32)
    for j in range(K):
        S = sum((Fraction(float(v)) ** 2 for v in Xf[:, j]), Fraction(0))
        out[j] = np.float32(rn64_sqrt(S))
    return out


def masks_from_bits(bits: np.ndarray) -> np.ndarray:
    """bool [R, K] -> uint32 [R, K/32], column 32w+b -> bit b of word w."""
    bits = np.asarray(bits, dtype=bool)
    R, K = bits.shape
    b = bits.reshape(R, K // 32, 32).astype(np.uint64)
    return (b << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
