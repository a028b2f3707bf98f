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


@pytest.mark.parametrize("ntiles,waves", [(1, 1), (63, 2), (64 * 5 + 3, 7), (100_000, 1024)])
def test_tile_probe_reads_every_listed_tile(lib, ntiles, waves):
    """The scattered-tile probe folds in every word of every listed tile once
    (a tile listed twice cancels), whatever the stretch each wavefront gets;
    out-of-range tile numbers are clamped into the buffer."""
    ntotal = 4096
    g = torch.Generator(device="cpu").manual_seed(ntiles)
    host = torch.randint(0, 256, (ntotal * 2048,), dtype=torch.uint8, generator=g)
    ids = torch.randint(0, ntotal, (ntiles,), dtype=torch.int32, generator=g)
    if ntiles > 10:
        ids[3] = -5                                      # clamped to tile 0
        ids[7] = ntotal + 9                              # clamped to the last tile
    data, tiles = host.to("cuda"), ids.to("cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.read_tiles_probe(data, tiles, sink, waves=waves)
    words = host.numpy().view(np.uint32).reshape(ntotal, 512)
    clamped = np.clip(ids.numpy(), 0, ntotal - 1)
    want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(words[clamped], axis=1))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
