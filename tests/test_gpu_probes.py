"""The bandwidth reference kernels (streaming copy and streaming read) move or
read every byte they are given: checked exactly against numpy."""
import numpy as np
import pytest
import torch

from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_304_amd as m
    return m


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (3 << 20) + 48, 64 << 20])
def test_hbm_read_folds_every_unit(m, nbytes):
    say(f"hbm_read {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((2048, 4), 0x5A5A5A5A, dtype=torch.int32, device="cuda")  # every unit is overwritten
    m.hbm_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32), axis=0)
    want = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nbytes", [1, 17, (1 << 20) + 7, 64 << 20])
def test_hbm_copy_copies_every_byte(m, nbytes):
    say(f"hbm_copy {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, size=nbytes, dtype=np.uint8)).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    m.hbm_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert not dst[nbytes:].any()  # nothing written past the end
