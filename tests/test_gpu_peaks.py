"""The measurement utilities behind the benchmark's measured ceilings
(dflash2_peak_mfma, dflash2_peak_read) run and return well-defined results:
zero operands give exactly zero sums, random ones finite non-zero sums, and
the streaming read's checksums are the XOR of the words each thread read."""
import numpy as np
import pytest
import torch

from block_speculative_decoding_dflash2_amd import _lib as L
from block_speculative_decoding_dflash2_amd.runner import current_stream

pytestmark = pytest.mark.gpu


def test_peak_mfma_runs():
    blocks = 8
    out = torch.full((blocks * 4,), float("nan"), dtype=torch.float32, device="cuda")
    L.dflash2_peak_mfma(current_stream(), blocks, 10, 1, out.data_ptr())
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    L.dflash2_peak_mfma(current_stream(), blocks, 10, 0, out.data_ptr())
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.any(o != 0)


def test_peak_read_checksums():
    blocks, n16 = 4, 4 * 256 * 5 + 3          # a ragged tail past the unrolled rounds
    words = np.random.default_rng(0).integers(0, 2**31, n16 * 4, dtype=np.int64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    L.dflash2_peak_read(current_stream(), src.data_ptr(), n16 * 16, blocks, out.data_ptr())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    w4 = words.reshape(n16, 4)
    per_word = w4[:, 0] ^ w4[:, 1] ^ w4[:, 2] ^ w4[:, 3]
    nthr = blocks * 256
    want = np.zeros(nthr, dtype=np.uint32)
    for t in range(nthr):
        want[t] = np.bitwise_xor.reduce(per_word[t::nthr]) if t < n16 else 0
    assert np.array_equal(got, want)
    with pytest.raises(L.DFlash2Error):
        L.dflash2_peak_read(current_stream(), src.data_ptr() + 4, 64, blocks, out.data_ptr())
