"""The measurement probes of include/fa_probe.h run through the C ABI on the GPU.

The read sweep XORs every 16-byte chunk it reads into its thread's sink word;
the XOR of all sink words must equal the XOR of all 32-bit words of the
buffer, which holds only if every byte is read exactly once.
"""
import numpy as np
import pytest
import torch

from io_aware_tiled_fwd_amd import binding

pytestmark = pytest.mark.gpu


def test_hbm_read_probe_reads_every_chunk_once():
    n = 2 * binding.PROBE_READ_UNIT // 4
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.empty(256 * 512, dtype=torch.int32, device="cuda")
    binding.fa_probe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words)
    assert got == want


def test_mfma_probe_runs():
    blocks = 8
    sink = torch.full((blocks * 512,), float("nan"), device="cuda")
    binding.fa_probe_mfma(blocks, 4, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
