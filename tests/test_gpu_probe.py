"""The streaming read probe (a diagnostic the bench reports beside the decode bandwidth) reads every
16-byte word once: each workgroup's xor of its words matches the host's."""

import numpy as np
import pytest
import torch

from mla_decode_paged_split_amd import binding

pytestmark = pytest.mark.gpu

WORDS_PER_GROUP = binding.MLA_READ_PROBE_BYTES_PER_WORD // 16  # 16-byte words each workgroup reads


def expected_sink(words: np.ndarray) -> np.ndarray:
    """Per-workgroup xor: workgroup k reads 16-byte words [k * WORDS_PER_GROUP, (k + 1) * WORDS_PER_GROUP)."""
    w16 = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1)
    groups = -(-w16.size // WORDS_PER_GROUP)
    out = np.zeros(groups, dtype=np.uint32)
    np.bitwise_xor.at(out, np.arange(w16.size) // WORDS_PER_GROUP, w16)
    return out


@pytest.mark.parametrize("n16", [WORDS_PER_GROUP * 4096 + 1234, WORDS_PER_GROUP * 3, WORDS_PER_GROUP + 1, 77, 1])
def test_read_probe_reads_every_word(gpu, n16):
    g = torch.Generator().manual_seed(n16)
    words = torch.randint(0, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = words.to(gpu)
    groups = binding.read_probe_sink_words(n16 * 16)
    sink = torch.full((groups + 8,), -1, dtype=torch.int32, device=gpu)
    binding.mla_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:groups], expected_sink(words.numpy().view(np.uint32)))
    assert np.all(got[groups:] == np.uint32(0xFFFFFFFF))  # nothing past the last workgroup's word


def test_read_probe_rejects_bad_sizes(gpu):
    sink = torch.zeros(4, dtype=torch.int32, device=gpu)
    with pytest.raises(Exception):
        binding.mla_read_probe(torch.zeros(20, dtype=torch.uint8, device=gpu), sink)  # not a multiple of 16
    with pytest.raises(Exception):  # five workgroups, four sink words
        binding.mla_read_probe(torch.zeros(4 * binding.MLA_READ_PROBE_BYTES_PER_WORD + 16, dtype=torch.uint8,
                                           device=gpu), sink)
