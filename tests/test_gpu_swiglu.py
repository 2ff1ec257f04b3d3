"""GPU parity of the gated-MLP launches (nm_spmv_swiglu, dense_gemv_swiglu) against the
oracle: h = silu(g) * u on fp64 oracle products, held to the bound a result inherits
from the matvec tolerance of g and u (oracle.swiglu_tolerance)."""
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


def _assert_h(h_bits, g, ag, u, au, what):
    h = bf16_as_f64(h_bits)
    ref = oracle.swiglu(g, u)
    ok = np.abs(h - ref) <= oracle.swiglu_tolerance(g, ag, u, au)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside, e.g. {i}: gpu={h[i]} ref={ref[i]}")


SHAPES = [(256, 512), (1000, 4096), (513, 5120), (17, 8192), (3, 28672), (1, 32)]
# Larger launch forms of the gated-MLP kernel, each with the plan it must get (kernel 0
# word-per-lane / 1 tile, workgroup size): 1024-thread workgroups at B = 1/2 (rows of
# 8192 columns) and B = 4 (x allows two workgroups per CU), the tile kernel at B = 3 for a
# row of x beyond the word-per-lane LDS slice.
WIDE = [(2048, 8192, 1, (0, 1024)), (2048, 8192, 2, (0, 1024)), (1500, 8192, 4, (0, 1024)),
        (1100, 11264, 3, (1, 512))]


@pytest.mark.parametrize("R,K,B", [(R, K, B) for R, K in SHAPES for B in (1, 3, 8)] + [w[:3] for w in WIDE])
def test_swiglu_sparse_and_dense(R, K, B):
    p = nm.nm_spmv_plan(R, K, B, nm.NM_EPI_SWIGLU)
    say("swiglu", R, K, B, p)
    for wr, wk, wb, plan in WIDE:
        if (wr, wk, wb) == (R, K, B):
            assert (p["kernel"], p["threads"]) == plan
    n = oracle.col_norm(synth.calib_acts(K, 8, R, K))
    Wg, Wu = synth.weights(R, K, 8, 1, R, K), synth.weights(R, K, 8, 2, R, K)
    gm, gv = oracle.prune_pack(Wg, n, 4, 8)
    um, uv = oracle.prune_pack(Wu, n, 4, 8)
    x = synth.decode_x(B, K, 8, R, K, B)
    xd = dev_bf16(x)
    h = nm.nm_spmv_swiglu((dev_u32(gm), dev_bf16(gv)), (dev_u32(um), dev_bf16(uv)), xd)
    hd = nm.dense_gemv_swiglu(dev_bf16(Wg), dev_bf16(Wu), xd)
    torch.cuda.synchronize()
    g, ag = oracle.spmv(gm, gv, x, K, nthreads=4)
    u, au = oracle.spmv(um, uv, x, K, nthreads=4)
    _assert_h(host_bf16(h), g, ag, u, au, f"sparse R={R} K={K} B={B}")
    g, ag = oracle.dense(Wg, x, nthreads=4)
    u, au = oracle.dense(Wu, x, nthreads=4)
    _assert_h(host_bf16(hd), g, ag, u, au, f"dense R={R} K={K} B={B}")


def test_swiglu_large_gate_values_and_zero_up():
    """Large |g| drives silu to g or 0; u = 0 rows give exactly 0."""
    say("swiglu extremes")
    R, K = 64, 256
    Wg = np.zeros((R, K), np.float32)
    Wg[:, :8] = 8.0                     # g = +-64 with x = +-1 in the first columns
    Wg[1::2, :8] = -8.0
    Wu = np.zeros((R, K), np.float32)
    Wu[:32, 8:16] = 0.5
    Wgb, Wub = synth.to_bf16_bits(Wg), synth.to_bf16_bits(Wu)
    x = synth.to_bf16_bits(np.ones((1, K), np.float32))
    n = np.ones(K, np.float32)
    gm, gv = oracle.prune_pack(Wgb, n, 16, 32)
    um, uv = oracle.prune_pack(Wub, n, 16, 32)
    h = host_bf16(nm.nm_spmv_swiglu((dev_u32(gm), dev_bf16(gv)), (dev_u32(um), dev_bf16(uv)), dev_bf16(x)))
    torch.cuda.synchronize()
    hf = bf16_as_f64(h)[0]
    assert (hf[32:] == 0).all()
    assert (hf[0:32:2] == 64.0 * 4.0).all()  # silu(64) = 64 in fp32, u = 4
    assert (np.abs(hf[1:32:2]) < 1e-20).all()
