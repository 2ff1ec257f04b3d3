"""The entry point that allocates nothing (nm_spmv_noalloc) against nm_spmv: the same
product through the same kernels, with split-row partial sums in the library's fixed
per-device scratch instead of a caller workspace.  Two calls in a row, the second with a
smaller input (the scratch keeps the first call's contents), must each equal nm_spmv bit
for bit and the oracle within the matvec tolerance."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_as_f64, dev_bf16, dev_u32, host_bf16, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402


def _case(R, K, B, seed):
    W = synth.weights(R, K, 70, seed)
    mref, vref = oracle.prune_pack(W, oracle.col_norm(synth.calib_acts(K, 70, seed)), 8, 16)
    x = synth.decode_x(B, K, 70, seed, B)
    return mref, vref, x


def _check(mref, vref, x, what):
    R, K, B = mref.shape[0], mref.shape[1] * 32, x.shape[0]
    m, v, xd = dev_u32(mref), dev_bf16(vref), dev_bf16(x)
    y_ref_call = nm.nm_spmv(m, v, xd)
    out = torch.full((B, R), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = nm.nm_spmv_noalloc(m, v, xd, out=out)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    assert (host_bf16(y) == host_bf16(y_ref_call)).all(), f"{what}: differs from nm_spmv"
    yref, absum = oracle.spmv(mref, vref, x, K)
    ok = oracle.within_tolerance(bf16_as_f64(host_bf16(y)), yref, absum)
    assert ok.all(), f"{what}: {int((~ok).sum())} outside tolerance"


@pytest.mark.parametrize("first,second", [((17, 8192, 1), (5, 4096, 2)), ((64, 28672, 2), (3, 8192, 1))])
def test_noalloc_matches_nm_spmv_on_two_calls(first, second):
    """Both shapes split their rows (partial sums in the scratch); the second is smaller."""
    say("noalloc", first, second)
    for R, K, B in (first, second):
        assert nm.nm_spmv_plan(R, K, B)["workspace_bytes"] > 0
    a, b = _case(*first, 1), _case(*second, 2)
    _check(*a, f"first {first}")
    _check(*b, f"second {second}")
    _check(*a, f"first again {first}")


@pytest.mark.parametrize("R,K,B,kind", [(1024, 4096, 1, 0), (512, 4096, 8, 1), (4096, 14336, 1, 2), (4160, 14336, 1, 3)])
def test_noalloc_without_split_rows(R, K, B, kind):
    """Shapes that need no scratch: whole rows, the matrix-core path at B = 8, and the
    one-token half-row and strip walks."""
    say("noalloc no split", R, K, B)
    p = nm.nm_spmv_plan(R, K, B)
    assert p["workspace_bytes"] == 0 and p["kernel"] == kind
    _check(*_case(R, K, B, 3), f"{R}x{K} B={B}")
