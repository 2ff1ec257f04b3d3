"""The streaming-read measurement kernel (nm_stream_read) reads every byte once: the XOR
of its per-wave folds equals the XOR of all dwords of the buffer (numpy on the
host, or a closed form for the 2^31-byte maximum)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a HIP GPU", allow_module_level=True)

import bitmask_spmv_amd as nm  # noqa: E402


def xor_all(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32).ravel()))


@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, 512 * 64 + 16, 512 * 64 * 1024 * 3 + 16, (1 << 20) + 32, 100 << 20])
def test_fold_equals_xor_of_all_dwords(nbytes):
    say("stream read", nbytes)
    g = np.random.default_rng(nbytes)
    host = g.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = nm.nm_stream_read(buf)
    torch.cuda.synchronize()
    assert sink.numel() == nm.nm_stream_read_sink_words(nbytes)
    assert xor_all(sink.cpu().numpy()) == xor_all(host)


def test_largest_buffer_closed_form():
    """2^31 bytes holding 1, 2, ..., 2^29: the XOR of 1..n is n when n % 4 == 0."""
    n = 1 << 29
    say("stream read max", 4 * n)
    buf = torch.arange(1, n + 1, dtype=torch.int32, device="cuda")
    sink = nm.nm_stream_read(buf)
    torch.cuda.synchronize()
    assert sink.numel() == 256 * 8  # 256 workgroups of 8 waves
    assert xor_all(sink.cpu().numpy()) == n
    del buf


def test_repeat_calls_agree_and_reuse_the_sink():
    buf = torch.randint(-(1 << 31), 1 << 31, (3 << 18,), dtype=torch.int32, device="cuda")
    s1 = nm.nm_stream_read(buf)
    s2 = nm.nm_stream_read(buf, sink=torch.full_like(s1, 7))
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
