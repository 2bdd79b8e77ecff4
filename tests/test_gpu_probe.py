"""The read-ceiling probe (kv8_read_probe, a measurement utility) reads the
bytes it claims: for a small buffer of random words and a random tile order,
each thread's xor of its eight 16-byte reads equals the host's."""
import numpy as np
import pytest
import torch

from paged_int8_kv_amd import binding as B
from tests.kv8_testutil import dev, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("tile_bytes", [2048, 4096, 32768])
def test_read_probe_reads_the_tiles(tile_bytes):
    rng = np.random.Generator(np.random.PCG64(5))
    n_tiles = 4 * 32768 // tile_bytes * 3            # room for three workgroups' worth, x4
    words = rng.integers(0, 2**32, size=n_tiles * tile_bytes // 4, dtype=np.uint32)
    per_wg = B.load().kv8_read_probe_bytes_per_workgroup()
    wg = 3
    order = rng.permutation(n_tiles)[: wg * per_wg // tile_bytes].astype(np.int32)
    buf = torch.from_numpy(words.view(np.uint8)).to(dev())
    out = torch.zeros(wg * 256, dtype=torch.int32, device=dev())
    read = B.kv8_read_probe(buf, torch.from_numpy(order).to(dev()), tile_bytes, out)
    torch.cuda.synchronize()
    assert read == wg * per_wg
    u4 = words.reshape(-1, 4)
    tile_u4 = tile_bytes // 16
    expect = np.zeros(wg * 256, np.uint32)
    for blk in range(wg):
        for i in range(8):
            p = blk * 2048 + i * 256 + np.arange(256)
            rows = order[p // tile_u4].astype(np.int64) * tile_u4 + p % tile_u4
            expect[blk * 256:(blk + 1) * 256] ^= np.bitwise_xor.reduce(u4[rows], axis=1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), expect)
