"""kv8_rope_quant_append on the GPU: the rotated, quantised K and the
quantised V bit-exact with the oracle's rope_quant_append (both head dims,
outlier channels, positions across a 128K table, clamped positions), the
identity at position 0, and decode over the fused cache against the
oracle."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B
from paged_int8_kv_amd import workloads as W
from tests.kv8_testutil import (bits_tensor, check_close, dev, download_cache, gpu_append,
                                gpu_decode, needs_gpu)
from tests.test_gpu_append import assert_cache_equal

pytestmark = [pytest.mark.gpu, needs_gpu]


def gpu_rope_append(case, positions, table):
    cache = B.alloc_cache(case.num_blocks, case.num_kv_heads, case.head_dim, dev())
    k = bits_tensor(case.k_bits).view(torch.bfloat16)
    v = bits_tensor(case.v_bits).view(torch.bfloat16)
    B.kv8_rope_quant_append(k, v, torch.from_numpy(case.slot_mapping).to(dev()),
                            torch.from_numpy(np.asarray(positions, np.int32)).to(dev()),
                            torch.from_numpy(table).to(dev()), *cache)
    return cache


def oracle_rope_cache(case, positions, table):
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, case.num_kv_heads, case.head_dim)
    O.rope_quant_append(case.k, case.v, positions, table, case.slot_mapping, kc, vc, ks, vs)
    return kc, vc, ks, vs


@pytest.mark.parametrize("hkv,d,offset", [(8, 128, 0), (8, 128, 120000), (2, 64, 37), (4, 128, 5)])
def test_rope_append_bitexact(hkv, d, offset):
    case = W.make_paged_case(batch=6, num_q_heads=hkv * 4, num_kv_heads=hkv, head_dim=d,
                             context_lens=[1, 15, 16, 17, 300, 1000], k_outliers=True,
                             seed=80 + d + offset % 7)
    table = W.rope_cos_sin(131072, d)
    pos = case.token_pos + offset
    got = download_cache(gpu_rope_append(case, pos, table))
    assert_cache_equal(got, oracle_rope_cache(case, pos, table), f"rope append d={d}")


def test_rope_append_clamps_positions():
    case = W.make_paged_case(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             context_lens=[40, 9], seed=85)
    table = W.rope_cos_sin(64, 128)
    pos = case.token_pos.astype(np.int64) * 3 - 20         # negative and past the table
    got = download_cache(gpu_rope_append(case, pos, table))
    exp = oracle_rope_cache(case, np.clip(pos, 0, 63), table)
    assert_cache_equal(got, exp, "clamped positions")


def test_rope_append_at_position_zero_is_plain_append():
    case = W.llama8b_decode(batch=3)
    table = W.rope_cos_sin(8, 128)
    got = download_cache(gpu_rope_append(case, np.zeros(len(case.slot_mapping)), table))
    plain = download_cache(gpu_append(case))
    assert_cache_equal(got, plain, "position 0")


def test_decode_over_rope_cache():
    """Append with RoPE at the tokens' positions, then decode: matches the
    oracle's decode over the oracle's fused cache."""
    case = W.llama8b_decode(batch=4)
    table = W.rope_cos_sin(8192, 128)
    cache = gpu_rope_append(case, case.token_pos, table)
    host = oracle_rope_cache(case, case.token_pos, table)
    assert_cache_equal(download_cache(cache), host, "fused cache")
    out = gpu_decode(case, cache)
    ref = O.paged_decode(case.q, *host, case.block_table, case.context_lens)
    check_close(out, ref, "decode over the fused cache")
