"""The peak probes the benchmark reports measured rates with do the work they are timed
for: the copy copies, the read's XOR covers every byte, and the MFMA loops' accumulators
end at exactly K * iters (all-ones operands)."""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_indexer_amd import peaks
from tests.dsa_dev import DEV

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_stream_copy_and_read():
    L = peaks.load()
    n16, blocks = 100003, 37                       # ragged: grid-stride tail
    rng = np.random.default_rng(0)
    host = rng.integers(0, 2 ** 32, n16 * 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    dst = torch.zeros_like(src)
    assert L.dsa_peak_stream_copy(src.data_ptr(), dst.data_ptr(), n16, blocks, _stream()) == 0
    out = torch.zeros(blocks * 4, dtype=torch.int32, device=DEV)
    assert L.dsa_peak_stream_read(src.data_ptr(), n16, blocks, out.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    x = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert x == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("fp8,K", [(0, 16), (1, 64)])
def test_mfma_loop_sums(fp8, K):
    L = peaks.load()
    blocks, iters = 5, 37
    res = torch.full((blocks * 4 * 2,), -1.0, dtype=torch.float32, device=DEV)
    assert L.dsa_peak_mfma(fp8, iters, blocks, res.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert (res.cpu() == float(K * iters)).all()
