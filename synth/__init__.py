"""Seeded synthetic inputs shared by the CPU oracle checks, the GPU parity tests and
the benchmark.

This module only draws random numbers and rounds them to the storage types the
library consumes (bfloat16 bit patterns, float32).  It holds none of the method's
arithmetic: no scores, no norms, no selection, no packing, no products.  Both the
oracle side and the HIP side receive exactly these arrays as inputs.

Distributions follow the synthetic stand-ins for the decode layers of Llama/Qwen
models (the pages measure end-to-end decode of real checkpoints, which are not
available here):

* weights      W = bf16_rne(0.02 * N(0, 1))                       [R, K]
* calibration  X = bf16_rne(N(0, 1) * s_j), s_j = exp(N(0, 1))     [T, K], T = 16
  (per-channel lognormal scale, so a few input channels dominate the norms, the
  way outlier channels do in trained models)
* decode input x = bf16_rne(N(0, 1))                               [B, K]

Host generators use numpy's PCG64 keyed by a SeedSequence over
(seed, *ids); device generators (throughput-only buffers of several GB) use a
torch CUDA generator seeded per buffer.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng", "to_bf16_bits", "bf16_bits_to_f32", "weights", "calib_acts",
    "decode_x", "ternary", "tie_stress", "device_weights", "device_calib_acts",
    "device_decode_x", "CALIB_TOKENS", "WEIGHT_STD",
]

CALIB_TOKENS = 16
WEIGHT_STD = 0.02


def rng(seed: int, *ids: int) -> np.random.Generator:
    """PCG64 stream keyed by (seed, *ids)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, ids)])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and return
    the raw 16-bit patterns as uint16.  Inputs must be finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def weights(R: int, K: int, seed: int = 0, *ids: int, std: float = WEIGHT_STD) -> np.ndarray:
    g = rng(seed, 1, *ids)
    return to_bf16_bits((std * g.standard_normal((R, K))).astype(np.float32))


def calib_acts(K: int, seed: int = 0, *ids: int, T: int = CALIB_TOKENS) -> np.ndarray:
    g = rng(seed, 2, *ids)
    scale = np.exp(g.standard_normal(K))
    return to_bf16_bits((g.standard_normal((T, K)) * scale[None, :]).astype(np.float32))


def decode_x(B: int, K: int, seed: int = 0, *ids: int) -> np.ndarray:
    g = rng(seed, 3, *ids)
    return to_bf16_bits(g.standard_normal((B, K)).astype(np.float32))


def ternary(shape, seed: int = 0, *ids: int) -> np.ndarray:
    """Values in {-1, 0, +1} as bf16 patterns (every partial sum of products of
    such values is a small integer, exactly representable in bf16 up to 256)."""
    g = rng(seed, 4, *ids)
    return to_bf16_bits(g.integers(-1, 2, size=shape).astype(np.float32))


def ternary_sparse(shape, density: float, seed: int = 0, *ids: int) -> np.ndarray:
    """Like ternary, with each entry kept nonzero only with probability `density`: long
    rows whose sums of products still stay small integers (bf16-exact up to 256)."""
    g = rng(seed, 6, *ids)
    v = g.integers(-1, 2, size=shape).astype(np.float32)
    v[g.random(size=shape) >= density] = 0.0
    return to_bf16_bits(v)


def tie_stress(R: int, K: int, seed: int = 0, *ids: int):
    """Weights drawn from {0, +-2^-4, +-2^-3} (and -0.0) and column norms from {1, 2}:
    many exactly equal scores inside every group, so the tie rule decides."""
    g = rng(seed, 5, *ids)
    pool = np.array([0.0, -0.0, 2.0 ** -4, -(2.0 ** -4), 2.0 ** -3, -(2.0 ** -3)], dtype=np.float32)
    W = to_bf16_bits(pool[g.integers(0, len(pool), size=(R, K))])
    n = np.array([1.0, 2.0], dtype=np.float32)[g.integers(0, 2, size=K)]
    return W, n


# ---------------------------------------------------------------- device side
def _torch_gen(seed: int, *ids: int):
    import torch

    ss = np.random.SeedSequence([int(seed), *map(int, ids)])
    s = int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))
    g = torch.Generator(device="cuda")
    g.manual_seed(s)
    return g


def device_weights(R: int, K: int, seed: int, *ids: int, std: float = WEIGHT_STD):
    """bf16 [R, K] on the current CUDA device (throughput-only buffers)."""
    import torch

    g = _torch_gen(seed, 11, *ids)
    w = torch.randn((R, K), generator=g, device="cuda", dtype=torch.float32)
    return (w * std).to(torch.bfloat16)


def device_calib_acts(K: int, seed: int, *ids: int, T: int = CALIB_TOKENS):
    import torch

    g = _torch_gen(seed, 12, *ids)
    scale = torch.exp(torch.randn((K,), generator=g, device="cuda", dtype=torch.float32))
    X = torch.randn((T, K), generator=g, device="cuda", dtype=torch.float32) * scale[None, :]
    return X.to(torch.bfloat16)


def device_decode_x(B: int, K: int, seed: int, *ids: int):
    import torch

    g = _torch_gen(seed, 13, *ids)
    return torch.randn((B, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
