"""The bandwidth probe reads every byte: its checksum is the XOR of all 32-bit
words of the buffer, computed here on the host."""
import numpy as np
import pytest
import torch

from tests.gpu_common import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


@pytest.mark.parametrize("words", [0, 4, 1028, (3 << 18) + 12, 1 << 26])
def test_read_probe_checksum(ps, words):
    g = torch.Generator(device="cpu").manual_seed(words)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (words,), generator=g, dtype=torch.int32)
    src = host.cuda()
    out = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    ps.ps_read_probe(src, out)
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32))) if words else 0
    assert int(out.cpu().numpy().view(np.uint32)[0]) == want
