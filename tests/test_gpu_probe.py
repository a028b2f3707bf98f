"""The read-bandwidth probe reads every byte it is given: its XOR of all
32-bit words equals the host's, for sizes that leave every kind of tail."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, (64 << 20) + 16 * 7])
def test_probe_reads_every_word(lib, nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    data = host.to("cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.read_bandwidth_probe(data, sink)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
    lib.read_bandwidth_probe(data, sink)                 # twice: XOR back to zero
    assert int(sink.cpu()[0]) == 0
