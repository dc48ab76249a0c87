"""The streaming-read probe (libmla_probe) reads every byte once: the XOR of
the words it leaves in its sink equals the XOR of all 32-bit words of the
buffer, for sizes that leave ranges partly filled or empty."""

from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, 4 * 1_000_003, 4 * 512 * 4096 + 12, 150_000_000])
def test_probe_reads_every_word(n_words):
    from mla_latent_kv_06_amd import binding as b
    print("[gpu-case] probe_read words", n_words, flush=True)
    g = torch.Generator().manual_seed(n_words)
    host = torch.randint(-2**31, 2**31 - 1, (n_words,), dtype=torch.int32, generator=g)
    buf = host.cuda()
    sink = torch.full((b.PROBE_SINK_BYTES,), 0x5A, dtype=torch.uint8, device="cuda")
    b.probe_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().view(torch.int32).numpy())
    want = np.bitwise_xor.reduce(host.numpy())
    assert got == want
