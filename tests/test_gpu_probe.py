"""The read-ceiling kernels (measurement utilities) read the bytes they
claim, for a small buffer of random words.  kv8_stream_read: each
persistent workgroup's threads xor exactly the 16-byte units of the chunks
they own (chunks w, w + workgroups, ...), with more chunks than workgroups
and with fewer.  kv8_read_probe: each wave xors the 1 KB rows of the tiles
it owns (list entries v, v + waves, ...), lane l unit l of each row, for
random tile orders, with fewer tiles than waves, and with more than 64
tiles per wave (several batches of tile ids)."""
import numpy as np
import pytest
import torch

from paged_int8_kv_amd import binding as B
from tests.kv8_testutil import dev, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

THREADS, ITERS = 256, 8
CHUNK_U4 = THREADS * ITERS


def expected(u4_rows_of_chunk, n_chunks, workgroups, words):
    u4 = words.reshape(-1, 4)
    x = np.bitwise_xor.reduce(u4, axis=1)
    exp = np.zeros(workgroups * THREADS, np.uint32)
    for c in range(n_chunks):
        w = c % workgroups
        rows = u4_rows_of_chunk(c)                      # [CHUNK_U4], position p = i*256 + t
        exp[w * THREADS:(w + 1) * THREADS] ^= np.bitwise_xor.reduce(
            x[rows].reshape(ITERS, THREADS), axis=0)
    return exp


@pytest.mark.parametrize("tile_bytes,n_read,workgroups", [
    (1024, 600, 1), (2048, 1000, 2), (2048, 37, 3), (4096, 5, 8), (32768, 9, 2)])
def test_read_probe_reads_the_tiles(tile_bytes, n_read, workgroups):
    rng = np.random.Generator(np.random.PCG64(5))
    n_tiles = 4 * n_read                                 # a buffer four times what is read
    words = rng.integers(0, 2**32, size=n_tiles * tile_bytes // 4, dtype=np.uint32)
    order = rng.permutation(n_tiles)[:n_read].astype(np.int32)
    buf = torch.from_numpy(words.view(np.uint8)).to(dev())
    out = torch.zeros(workgroups * THREADS, dtype=torch.int32, device=dev())
    read = B.kv8_read_probe(buf, torch.from_numpy(order).to(dev()), tile_bytes, workgroups, out)
    torch.cuda.synchronize()
    assert read == n_read * tile_bytes
    x = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1)     # per 16-byte unit
    waves, tile_u4 = workgroups * THREADS // 64, tile_bytes // 16
    exp = np.zeros(workgroups * THREADS, np.uint32)
    for i, t in enumerate(order):
        v = i % waves                                   # the wave that reads list entry i
        for k in range(tile_bytes // 1024):
            exp[64 * v:64 * (v + 1)] ^= x[int(t) * tile_u4 + 64 * k + np.arange(64)]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), exp)


@pytest.mark.parametrize("n_chunks,workgroups", [(9, 4), (2, 6)])
def test_stream_read_reads_the_buffer(n_chunks, workgroups):
    rng = np.random.Generator(np.random.PCG64(6))
    words = rng.integers(0, 2**32, size=n_chunks * CHUNK_U4 * 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.uint8)).to(dev())
    out = torch.zeros(workgroups * THREADS, dtype=torch.int32, device=dev())
    assert B.kv8_stream_read(buf, workgroups, out) == n_chunks * CHUNK_U4 * 16
    torch.cuda.synchronize()
    rows = lambda c: c * CHUNK_U4 + np.arange(CHUNK_U4)
    assert np.array_equal(out.cpu().numpy().view(np.uint32),
                          expected(rows, n_chunks, workgroups, words))
