"""The read probe (a measurement aid for the decode roofline) reads every
word of its buffer exactly once: the XOR of the per-workgroup words it
writes equals the XOR of the buffer's 32-bit words."""
import numpy as np
import pytest
import torch

import paged_kv_attention_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, 300 << 20])
def test_read_probe_reads_every_word_once(nbytes):
    g = torch.Generator().manual_seed(nbytes % 1000)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to("cuda")
    sink = torch.full((pa.READ_PROBE_SINK_BYTES // 4,), -1, dtype=torch.int32, device="cuda")
    pa.read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
