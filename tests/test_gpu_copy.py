"""GPU: the library's streaming copy (ssq_stream_copy) copies bytes exactly, through the C ABI.

It is the bandwidth reference the bench compares a step with, so it must move every byte:
sizes below one workgroup, a ragged last workgroup and a large buffer."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mamba_decode_amd as ssq


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 48, (1 << 20) + 16 * 7, 64 << 20])
def test_stream_copy_is_exact(nbytes):
    print(f"stream copy {nbytes} bytes", file=sys.stderr, flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, size=nbytes + 64, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    ssq.ssq_stream_copy(dst, src, nbytes)
    out = dst.cpu().numpy()
    assert np.array_equal(out[:nbytes], host[:nbytes])
    assert not out[nbytes:].any()  # nothing beyond the requested bytes


def test_stream_copy_zero_bytes_and_errors():
    src = torch.ones(64, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(64, dtype=torch.uint8, device="cuda")
    ssq.ssq_stream_copy(dst, src, 0)
    torch.cuda.synchronize()
    assert not dst.cpu().numpy().any()
    with pytest.raises(ssq.SsqError) as e:
        ssq.ssq_stream_copy(dst, src, 24)
    assert e.value.status == ssq.SSQ_ERR_INVALID_ARG
    with pytest.raises(ssq.SsqError):
        ssq.ssq_stream_copy(src, src, 64)  # overlapping
