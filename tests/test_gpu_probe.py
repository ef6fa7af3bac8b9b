"""The pure-read bandwidth probe reads every byte it is given: the XOR it
leaves behind must equal the XOR of all 32-bit words of the buffer, computed
on the host, for sizes that end inside a thread's and a workgroup's share."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


@pytest.mark.parametrize("nbytes", [16, 4096, 32768 + 16, 1 << 20, (1 << 22) + 48])
def test_read_probe_reads_every_word(ops, nbytes):
    g = np.random.default_rng(nbytes)
    host = g.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops._lib.call("wsx_read_probe", ops._p(buf), nbytes, ops._p(out), ops._stream())
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want)
