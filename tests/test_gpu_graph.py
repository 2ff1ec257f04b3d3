"""The library's launches captured in a HIP graph, as a decode engine (and bench.py) runs
them: every replay must give, bit for bit, what the same calls give eagerly on the
inputs present at replay time.  Covers the word-per-lane kernel (plain, multi-matrix,
gated MLP, split rows with the workspace and the second pass), the matrix-core path at
B = 8 and the dense baseline.  Between replays the inputs are overwritten in place and
eager work runs on the stream, so a replay that reused stale results or depended on
state left by an earlier launch would show."""
from __future__ import annotations

import pytest
import torch

import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402


def _pack(R, K, *ids, N=2, M=4):
    W = synth.device_weights(R, K, 0, 70, R, K, *ids)
    n = nm.nm_col_norm(synth.device_calib_acts(K, 0, 71, K, *ids))
    return nm.nm_prune_pack(W, n, N, M)


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


@pytest.mark.parametrize("B", [1, 3, 8])
def test_graph_replays_match_eager(B):
    say("graph replays", B)
    K, K2 = 4096, 14336
    q, k, v = _pack(512, K, 1), _pack(128, K, 2), _pack(128, K, 3)
    g, u = _pack(1024, K, 4, N=8, M=16), _pack(1024, K, 5, N=8, M=16)
    down = _pack(64, K2, 6, N=16, M=32)  # few rows, wide: split rows at B <= 4
    # one token: half rows (4096 rows of 7 strips) and strips (4160 rows) per wave
    hr, st = _pack(4096, K2, 7), _pack(4160, K2, 8, N=4, M=8)
    Wd = synth.device_weights(256, K, 0, 72, B)
    x = synth.device_decode_x(B, K, 0, 73, B)
    x2 = synth.device_decode_x(B, K2, 0, 74, B)
    nbytes = max(nm.nm_spmv_multi_workspace_bytes([512, 128, 128], K, B), nm.nm_spmv_swiglu_workspace_bytes(1024, K, B),
                 nm.nm_spmv_workspace_bytes(64, K2, B), nm.dense_gemv_workspace_bytes(256, K, B),
                 nm.nm_spmv_workspace_bytes(4096, K2, B), nm.nm_spmv_workspace_bytes(4160, K2, B), 4)
    ws = torch.empty(nbytes // 4 + 1, dtype=torch.float32, device="cuda")
    outs = [torch.empty((B, r), dtype=torch.bfloat16, device="cuda") for r in (512, 128, 128)]
    h = torch.empty((B, 1024), dtype=torch.bfloat16, device="cuda")
    yd = torch.empty((B, 64), dtype=torch.bfloat16, device="cuda")
    yq = torch.empty((B, 512), dtype=torch.bfloat16, device="cuda")
    ydense = torch.empty((B, 256), dtype=torch.bfloat16, device="cuda")
    yh = torch.empty((B, 4096), dtype=torch.bfloat16, device="cuda")
    ys = torch.empty((B, 4160), dtype=torch.bfloat16, device="cuda")
    if B == 1:
        assert nm.nm_spmv_plan(4096, K2, 1)["kernel"] == nm.NM_KERNEL_WORD_HALF_ROWS
        assert nm.nm_spmv_plan(4160, K2, 1)["kernel"] == nm.NM_KERNEL_WORD_STRIPS

    def step():
        nm.nm_spmv_multi([q, k, v], x, outs=outs, workspace=ws)
        nm.nm_spmv(*q, x, out=yq, workspace=ws)
        nm.nm_spmv_swiglu(g, u, x, out=h, workspace=ws)
        nm.nm_spmv(*down, x2, out=yd, workspace=ws)
        nm.dense_gemv(Wd, x, out=ydense, workspace=ws)
        nm.nm_spmv(*hr, x2, out=yh, workspace=ws)
        nm.nm_spmv(*st, x2, out=ys, workspace=ws)

    def snapshot():
        return [t.clone() for t in (*outs, yq, h, yd, ydense, yh, ys)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # first calls (device queries, LDS attributes) outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        x.copy_(synth.device_decode_x(B, K, 0, 75, B, rep))
        x2.copy_(synth.device_decode_x(B, K2, 0, 76, B, rep))
        torch.cuda.synchronize()
        step()  # eager on the current stream
        torch.cuda.synchronize()
        want = snapshot()
        for t in (*outs, yq, h, yd, ydense, yh, ys):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        names = ["q", "k", "v", "q alone", "h", "down", "dense", "half rows", "strips"]
        for name, a, b in zip(names, got, want):
            assert _same(a, b), f"B={B} replay {rep}: {name} differs from the eager result"
