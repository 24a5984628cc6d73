"""GPU check of the read-stream measurement export: every byte is read exactly once, in the
documented thread order (sink value of thread t of workgroup g = XOR of the 16-byte chunks
its wave lane loads)."""

import numpy as np
import pytest
import torch

from tests.gpu_helpers import gpu, needs_gpu, say

pytestmark = [gpu, needs_gpu]


def test_read_stream_probe_reads_every_byte_once():
    from paged_kv_cascade_amd import api
    say("case: read_stream_probe over 3 MiB of int32 0..n-1")
    mib = 3
    n = mib * (1 << 20) // 4
    buf = torch.arange(n, dtype=torch.int32, device="cuda")
    sink = api.read_stream_probe(buf)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    # [workgroup, wave, load, lane, word]: wave w of workgroup g reads 256 KB from
    # (4g + w) * 256 KB; load i of lane l is the 16 bytes at 1 KB * i + 16 * l.
    v = np.arange(n, dtype=np.uint32).reshape(mib, 4, 256, 64, 4)
    want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(v, axis=4), axis=2)   # [g, w, lane]
    assert np.array_equal(got.reshape(mib, 4, 64), want)


def test_read_stream_probe_rejects_bad_sizes():
    from paged_kv_cascade_amd import api
    with pytest.raises(api.PkcError):
        api.read_stream_probe(torch.zeros(1000, dtype=torch.uint8, device="cuda"))
