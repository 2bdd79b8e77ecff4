"""paged_prefill_chunk_attn_kv8 on the GPU against the fp64 oracle (same
dequantised cache): ragged chunks over several query tiles and key tiles,
every supported group size and head dim, the full chunked-prefill shape on
sampled rows, and the invariants of the causal rule (locality, first row,
no visible key), block permutation, poisoned slots and determinism."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import workloads as W
from tests.kv8_testutil import (check_close, gpu_append, gpu_decode, gpu_prefill, needs_gpu,
                                oracle_cache, oracle_prefill_rows, upload_cache)

pytestmark = [pytest.mark.gpu, needs_gpu]


def oracle_full(case, cache_host, q=None, context_lens=None):
    kc, vc, ks, vs = cache_host
    return O.paged_prefill_chunk(case.q if q is None else q, case.extra["q_start_loc"],
                                 kc, vc, ks, vs, case.block_table,
                                 case.context_lens if context_lens is None else context_lens)


def run_parity(case, what):
    host = oracle_cache(case)
    out = gpu_prefill(case, upload_cache(*host))
    ref = oracle_full(case, host)
    check_close(out, ref, what)
    return out, ref, host


@pytest.mark.parametrize("hq,hkv,d", [
    (4, 1, 64), (8, 4, 64), (16, 2, 128), (64, 8, 128), (32, 8, 128), (8, 8, 128),
])
def test_prefill_ragged_group_sizes_and_dims(hq, hkv, d):
    """Chunks of 1, 77, 300 and 0 rows after 0, 5, 1000 and 17 earlier
    tokens: partial query tiles, partial key tiles, the causal diagonal
    inside and across tiles, an empty chunk."""
    case = W.prefill_case([0, 5, 1000, 17], [1, 77, 300, 0], num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=d, seed=hq * 3 + d, k_outliers=True)
    run_parity(case, f"prefill hq={hq} hkv={hkv} d={d}")


def test_prefill_chunked_config_reduced_batch():
    """The chunked-prefill shape (32/8 heads, d=128, 512-row chunks after
    2048..8192 tokens) at batch 2, every row checked."""
    case = W.chunked_prefill(batch=2)
    run_parity(case, "chunked prefill batch 2")


def test_prefill_chunked_config_full_sampled():
    """Full chunked-prefill shape (batch 8), cache built by the GPU append
    kernel, launched as the benchmark launches it; rows sampled across every
    sequence (first, tile edges, last, random) checked against the oracle."""
    case = W.chunked_prefill()
    host = oracle_cache(case)
    out = gpu_prefill(case, gpu_append(case))
    rng = np.random.default_rng(7)
    picks = []
    for b in range(case.batch):
        for i in sorted({0, 1, 63, 64, 255, 256, 511, *rng.integers(0, 512, 3).tolist()}):
            picks.append((b, int(i)))
    ref = oracle_prefill_rows(case, host, picks)
    qsl = case.extra["q_start_loc"]
    got = np.stack([out[qsl[b] + i] for b, i in picks])
    check_close(got, ref, "chunked prefill full, sampled rows")


def test_prefill_long_chunks_sampled():
    """Chunks of 4096 and 2049 rows after 0 and 12000 earlier tokens (64 and
    33 query tiles per KV head at G = 4): the longest causal diagonals and
    the most query tiles per pair.  Rows sampled at tile edges, the chunk's
    ends and at random, all query heads, against the oracle."""
    lens = [4096, 2049]
    case = W.prefill_case([0, 12000], lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                          seed=140, k_outliers=True)
    host = oracle_cache(case)
    out = gpu_prefill(case, upload_cache(*host))
    rng = np.random.default_rng(141)
    picks = []
    for b, n in enumerate(lens):
        rows = {0, 1, 63, 64, 127, 128, 1023, 1024, 2047, 2048, n - 2, n - 1,
                *rng.integers(0, n, 6).tolist()}
        picks += [(b, int(i)) for i in sorted(r for r in rows if 0 <= r < n)]
    ref = oracle_prefill_rows(case, host, picks)
    qsl = case.extra["q_start_loc"]
    got = np.stack([out[qsl[b] + i] for b, i in picks])
    check_close(got, ref, "long chunks, sampled rows")


def test_prefill_chunk_of_one_matches_decode():
    """A chunk of one row is a decode step: both kernels agree with the
    oracle's decode."""
    case = W.prefill_case([40, 700, 2000], [1, 1, 1], seed=41)
    host = oracle_cache(case)
    cache = upload_cache(*host)
    out = gpu_prefill(case, cache)
    ref = O.paged_decode(case.q, *host, case.block_table, case.context_lens)
    check_close(out, ref, "chunk of one vs oracle decode")
    dec = gpu_decode(case, cache, q=case.q_bits)
    check_close(dec, ref, "decode on the same case")


def test_prefill_causal_locality_bitwise():
    """Changing K/V of tokens after position p leaves every row at position
    <= p bitwise unchanged."""
    case = W.prefill_case([300, 64], [200, 100], seed=42)
    host = oracle_cache(case)
    out = gpu_prefill(case, upload_cache(*host))
    cut = {0: 300 + 120, 1: 64 + 37}       # last position kept per sequence
    kc, vc, ks, vs = (x.copy() for x in host)
    rng = np.random.default_rng(5)
    for b, p in cut.items():
        for t in range(p + 1, int(case.context_lens[b])):
            blk, off = int(case.block_table[b][t // 16]), t % 16
            kc[blk, :, off] = rng.integers(-127, 128, size=kc[blk, :, off].shape)
            vc[blk, :, off] = rng.integers(-127, 128, size=vc[blk, :, off].shape)
            ks[blk, :, off] = np.float16(rng.uniform(0.001, 1.0))
            vs[blk, :, off] = np.float16(rng.uniform(0.001, 1.0))
    out2 = gpu_prefill(case, upload_cache(kc, vc, ks, vs))
    qsl = case.extra["q_start_loc"]
    for b, p in cut.items():
        keep = p - int(case.extra["ctx_prev"][b]) + 1      # rows 0 .. keep-1
        a = out[qsl[b]:qsl[b] + keep]
        c = out2[qsl[b]:qsl[b] + keep]
        assert np.array_equal(a, c), f"sequence {b}: earlier rows changed"
        assert not np.array_equal(out[qsl[b] + keep:qsl[b + 1]], out2[qsl[b] + keep:qsl[b + 1]])


def test_prefill_first_row_sees_one_key_exactly():
    """With no earlier context, chunk row 0 sees only token 0: its output is
    that token's dequantised V exactly."""
    case = W.prefill_case([0, 0], [33, 300], num_q_heads=16, num_kv_heads=4, seed=43)
    out, ref, host = run_parity(case, "no earlier context")
    kc, vc, ks, vs = host
    qsl = case.extra["q_start_loc"]
    for b in range(2):
        for h in range(16):
            v0 = O.gather_dequant(vc, vs, case.block_table[b], 1, h // 4)[0]
            assert np.array_equal(out[qsl[b], h], v0.astype(np.float32))


def test_prefill_rows_without_visible_key_are_zero():
    """context_lens below the chunk length puts the first rows at negative
    positions; they see no key and come out as 0, the rest match the
    oracle."""
    case = W.prefill_case([100], [150], num_q_heads=8, num_kv_heads=2, seed=44)
    host = oracle_cache(case)
    ctx = np.array([120], np.int32)          # rows 0..29 at positions < 0
    out = gpu_prefill(case, upload_cache(*host), context_lens=ctx)
    assert np.all(out[:30] == 0)
    ref = oracle_prefill_rows(case, host, [(0, i) for i in range(30, 150)], context_lens=ctx)
    check_close(out[30:150], ref, "rows with visible keys")


def test_prefill_block_permutation_bitwise():
    base = W.prefill_case([500, 20, 1300], [130, 260, 64], seed=45, permute=False)
    host = oracle_cache(base)
    out = gpu_prefill(base, upload_cache(*host))
    perm = np.random.default_rng(4).permutation(base.num_blocks)
    arrs = []
    for a in host:
        p = np.empty_like(a)
        p[perm] = a
        arrs.append(p)
    out2 = gpu_prefill(base, upload_cache(*arrs), block_table=perm[base.block_table])
    assert np.array_equal(out, out2)


def test_prefill_poisoned_unused_slots():
    case = W.prefill_case([21, 70], [40, 9], num_q_heads=16, num_kv_heads=4, seed=46,
                          spare_blocks=3)
    kc, vc, ks, vs = oracle_cache(case)
    ref = oracle_full(case, (kc, vc, ks, vs))
    used = set()
    for b in range(2):
        for t in range(int(case.context_lens[b])):
            used.add((int(case.block_table[b][t // 16]), t % 16))
    for blk in range(case.num_blocks):
        for off in range(16):
            if (blk, off) not in used:
                kc[blk, :, off] = 127
                vc[blk, :, off] = -127
                ks[blk, :, off] = np.float16(np.nan)
                vs[blk, :, off] = np.float16(np.inf)
    out = gpu_prefill(case, upload_cache(kc, vc, ks, vs))
    check_close(out, ref, "poisoned")


def test_prefill_deterministic_and_context_cap():
    case = W.prefill_case([900, 3000, 50], [200, 120, 256], seed=47)
    host = oracle_cache(case)
    cache = upload_cache(*host)
    a = gpu_prefill(case, cache)
    b = gpu_prefill(case, cache)
    assert np.array_equal(a, b)
    cap = 2000          # clamps sequence 1 (3120 tokens) to 2000
    out = gpu_prefill(case, cache, max_context_len=cap)
    ref = oracle_full(case, host, context_lens=np.minimum(case.context_lens, cap))
    check_close(out, ref, "context cap")


def test_prefill_identical_keys_give_prefix_mean_v():
    case = W.prefill_case([10], [70], num_q_heads=8, num_kv_heads=2, seed=48)
    case.k[:] = case.k[0]
    case.k_bits[:] = case.k_bits[0]
    host = oracle_cache(case)
    kc, vc, ks, vs = host
    out = gpu_prefill(case, upload_cache(*host))
    for g in range(2):
        v = O.gather_dequant(vc, vs, case.block_table[0], 80, g)
        for i in (0, 13, 69):
            vm = v[:10 + i + 1].mean(0)
            for h in range(g * 4, g * 4 + 4):
                check_close(out[i, h], vm, "identical keys")


def test_prefill_large_logits_dominant_key():
    case = W.prefill_case([600], [64], num_q_heads=4, num_kv_heads=1, seed=49)
    host = oracle_cache(case)
    kc, vc, ks, vs = host
    kd = O.gather_dequant(kc, ks, case.block_table[0], 664, 0)
    q = np.zeros_like(case.q)
    q[:, :] = kd[123] * (3000.0 / np.dot(kd[123], kd[123]))
    qv, qb = W.to_bf16(q)
    out = gpu_prefill(case, upload_cache(*host), q=qb)
    ref = oracle_full(case, host, q=qv)
    check_close(out, ref, "dominant key")
