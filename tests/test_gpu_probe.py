"""The read-ceiling kernels (measurement utilities) read the bytes they
claim: for a small buffer of random words, each persistent workgroup's
threads xor exactly the 16-byte units of the chunks they own (chunks w,
w + workgroups, ...), for random tile orders (kv8_read_probe) and for the
contiguous stream (kv8_stream_read), with more chunks than workgroups and
with fewer."""
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


@pytest.mark.parametrize("tile_bytes,n_chunks,workgroups", [
    (256, 7, 3), (2048, 5, 5), (4096, 3, 8), (32768, 6, 4)])
def test_read_probe_reads_the_tiles(tile_bytes, n_chunks, workgroups):
    rng = np.random.Generator(np.random.PCG64(5))
    chunk = B.load().kv8_read_probe_chunk_bytes()
    assert chunk == CHUNK_U4 * 16
    n_read = n_chunks * chunk // tile_bytes
    n_tiles = 4 * n_read                                 # a buffer four times what is read
    words = rng.integers(0, 2**32, size=n_tiles * tile_bytes // 4, dtype=np.uint32)
    order = rng.permutation(n_tiles)[:n_read].astype(np.int32)
    buf = torch.from_numpy(words.view(np.uint8)).to(dev())
    out = torch.zeros(workgroups * THREADS, dtype=torch.int32, device=dev())
    read = B.kv8_read_probe(buf, torch.from_numpy(order).to(dev()), tile_bytes, workgroups, out)
    torch.cuda.synchronize()
    assert read == n_chunks * chunk
    tile_u4 = tile_bytes // 16

    def rows(c):
        p = c * CHUNK_U4 + np.arange(CHUNK_U4)
        return order[p // tile_u4].astype(np.int64) * tile_u4 + p % tile_u4
    assert np.array_equal(out.cpu().numpy().view(np.uint32),
                          expected(rows, n_chunks, workgroups, words))


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
