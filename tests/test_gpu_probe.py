"""GPU: the tile-read probe reads exactly the tiles it is given.

The xor of every thread's fold is the xor of every 32-bit word of the
tiles read (each tile read once), whatever the split over threads."""

import numpy as np
import pytest
import torch

import paged_kv_cache_29_amd as pkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("streaming", [False, True])
@pytest.mark.parametrize("ntiles,grid", [(3000, 64), (1, 1), (4096, 8), (517, 3)])
def test_probe_reads_the_named_tiles(ntiles, grid, streaming):
    rng = np.random.default_rng(ntiles)
    pool_tiles = 4096
    host = rng.integers(0, 2**32, size=pool_tiles * 1024, dtype=np.uint32)
    pool = torch.from_numpy(host.view(np.uint8)).to("cuda:0")
    ids = rng.choice(pool_tiles, size=ntiles, replace=False).astype(np.int32)
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda:0")
    pkv.probe_tile_read(pool, torch.from_numpy(ids).to("cuda:0"), sink, grid, streaming=streaming)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.reshape(pool_tiles, 1024)[ids].ravel())
    assert got == want


def test_probe_rejects_ids_outside_the_pool():
    pool = torch.zeros(8 * 4096, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    with pytest.raises(ValueError):
        pkv.probe_tile_read(pool, torch.tensor([0, 8], dtype=torch.int32, device="cuda:0"), sink, 1)
