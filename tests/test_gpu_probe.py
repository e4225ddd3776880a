"""The streaming read probe (a diagnostic the bench reports beside the decode bandwidth) reads every
16-byte word once: each workgroup's xor of its words matches the host's."""

import numpy as np
import pytest
import torch

from mla_decode_paged_split_amd import binding

pytestmark = pytest.mark.gpu

BLOCKS = binding.MLA_READ_PROBE_SINK_WORDS
THREADS = 256


def expected_sink(words: np.ndarray) -> np.ndarray:
    """Per-workgroup xor: workgroup k reads the k-th of BLOCKS equal contiguous shares of the 16-byte
    words; the words past the last whole share are read by thread (i - BLOCKS * share) of the grid."""
    w16 = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1)
    per = w16.size // BLOCKS
    idx = np.arange(w16.size)
    block = np.where(idx < BLOCKS * per, idx // max(per, 1), (idx - BLOCKS * per) // THREADS)
    out = np.zeros(BLOCKS, dtype=np.uint32)
    np.bitwise_xor.at(out, block, w16)
    return out


@pytest.mark.parametrize("n16", [BLOCKS * 4096 + 1234, BLOCKS * 3 + 200, 77])
def test_read_probe_reads_every_word(gpu, n16):
    g = torch.Generator().manual_seed(n16)
    words = torch.randint(0, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = words.to(gpu)
    sink = torch.full((BLOCKS,), -1, dtype=torch.int32, device=gpu)
    binding.mla_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_sink(words.numpy().view(np.uint32)))


def test_read_probe_rejects_bad_sizes(gpu):
    sink = torch.zeros(BLOCKS, dtype=torch.int32, device=gpu)
    with pytest.raises(Exception):
        binding.mla_read_probe(torch.zeros(20, dtype=torch.uint8, device=gpu), sink)  # not a multiple of 16
    with pytest.raises(Exception):
        binding.mla_read_probe(torch.zeros(64, dtype=torch.uint8, device=gpu), sink[:10])  # sink too small
