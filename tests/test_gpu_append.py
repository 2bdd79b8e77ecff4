"""kv8_quant_append on the GPU: int8 codes and fp16 scales bit-exact with
the oracle's quantiser, including exhaustive bf16 sweeps and edge rows."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import workloads as W
from tests.kv8_testutil import (dev, download_cache, gpu_append, needs_gpu, oracle_cache)

pytestmark = [pytest.mark.gpu, needs_gpu]


def assert_cache_equal(got, exp, what):
    names = ("k codes", "v codes", "k scales", "v scales")
    for n, g, e in zip(names, got, exp):
        if g.dtype == np.float16:
            g, e = g.view(np.uint16), np.asarray(e, np.float16).view(np.uint16)
        bad = np.argwhere(g != e)
        assert bad.size == 0, f"{what}: {n} differ at {len(bad)} places, first {bad[:3].tolist()}"


def rows_case(rows_k, rows_v, hkv=1):
    """Pack bf16 rows [N*hkv, d] into a case with identity slots."""
    rows_k = np.asarray(rows_k, np.float32)
    rows_v = np.asarray(rows_v, np.float32)
    n = rows_k.shape[0] // hkv
    d = rows_k.shape[1]
    kv, kb = W.to_bf16(rows_k.reshape(n, hkv, d))
    vv, vb = W.to_bf16(rows_v.reshape(n, hkv, d))
    nb = -(-n // 16)
    case = W.make_paged_case(batch=1, num_q_heads=hkv, num_kv_heads=hkv, head_dim=d,
                             context_lens=[1], seed=0)
    case.k, case.v, case.k_bits, case.v_bits = kv, vv, kb, vb
    case.num_blocks = nb
    case.slot_mapping = np.arange(n, dtype=np.int32)
    return case


@pytest.mark.parametrize("maker", [W.tiny_decode, W.llama8b_decode], ids=["tiny", "llama8b"])
def test_append_configs_bitexact(maker):
    case = maker()
    got = download_cache(gpu_append(case))
    assert_cache_equal(got, oracle_cache(case), maker.__name__)


def test_append_chunked_prefill_config_bitexact():
    case = W.chunked_prefill()
    got = download_cache(gpu_append(case))
    assert_cache_equal(got, oracle_cache(case), "chunked prefill")


def test_append_exhaustive_absmax():
    """Every positive finite bf16 value as the absmax of a row."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    a = W.bf16_bits_to_f32(bits)
    d = 64
    rng = np.random.default_rng(3)
    rows = (rng.uniform(-1, 1, size=(len(a), d)).astype(np.float32) * a[:, None])
    rows[:, 0] = a
    rows[np.arange(len(a)) % 2 == 1, 0] = -a[np.arange(len(a)) % 2 == 1]
    rows = W.to_bf16(rows)[0]
    rows[:, 0] = np.where(np.arange(len(a)) % 2 == 1, -a, a)    # absmax element exact
    case = rows_case(rows, rows[::-1].copy())
    got = download_cache(gpu_append(case))
    assert_cache_equal(got, oracle_cache(case), "absmax sweep")


@pytest.mark.parametrize("absmax", [127.0, 1.0, 0.0234375, 1e-4, 3e-6, 8323072.0, 3.0e38])
def test_append_exhaustive_values_for_scale(absmax):
    """Every finite bf16 x with |x| <= absmax, in rows whose absmax (hence
    scale) is fixed: normal, subnormal, zero and saturated scales."""
    a = float(W.to_bf16(np.array([absmax], np.float32))[0][0])
    allx = W.bf16_bits_to_f32(np.arange(0x10000, dtype=np.uint32).astype(np.uint16))
    x = allx[np.isfinite(allx) & (np.abs(allx) <= a)]
    d = 128
    per = d - 1
    n = -(-len(x) // per)
    pad = np.zeros(n * per, np.float32)
    pad[:len(x)] = x
    rows = np.concatenate([np.full((n, 1), a, np.float32), pad.reshape(n, per)], axis=1)
    case = rows_case(rows, -rows)
    got = download_cache(gpu_append(case))
    assert_cache_equal(got, oracle_cache(case), f"values under absmax {absmax}")


def test_append_edge_rows_ties_zero():
    d = 64
    s = 1.0
    ties = np.array([127.0] + [(k + 0.5) * s * (-1) ** k for k in range(-40, 23)], np.float32)
    rows = np.stack([ties, np.zeros(d, np.float32), np.full(d, 3.0e-6, np.float32),
                     np.full(d, -2.5, np.float32)])
    case = rows_case(rows, rows[::-1].copy())
    got = download_cache(gpu_append(case))
    assert_cache_equal(got, oracle_cache(case), "edge rows")


def test_append_skips_negative_and_out_of_range_slots():
    case = W.make_paged_case(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             context_lens=[30, 45], seed=14)
    slots = case.slot_mapping.copy()
    slots[[0, 7, 44]] = -1
    slots[[3, 50]] = case.num_blocks * 16 + 5        # beyond the cache: skipped
    kc_d = torch.full((case.num_blocks, 2, 16, 128), 0x5A, dtype=torch.int8, device=dev())
    ks_d = torch.full((case.num_blocks, 2, 16), 0x7C01, dtype=torch.int16, device=dev())
    cache = (kc_d, kc_d.clone(), ks_d, ks_d.clone())
    got = download_cache(gpu_append(case, cache=cache, slots=slots))
    kc = np.full((case.num_blocks, 2, 16, 128), 0x5A, np.int8)
    vc = kc.copy()
    ks_h = np.full((case.num_blocks, 2, 16), 0x7C01, np.int16).view(np.float16)
    vs_h = ks_h.copy()
    keep = slots.copy()
    keep[keep >= case.num_blocks * 16] = -1
    O.quant_append(case.k, case.v, keep, kc, vc, ks_h, vs_h)
    assert_cache_equal(got, (kc, vc, ks_h, vs_h), "skipped slots")


def test_append_twice_overwrites():
    case = W.make_paged_case(batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64,
                             context_lens=[40], seed=15)
    cache = gpu_append(case)
    k2 = case.k_bits[::-1].copy()
    v2 = case.v_bits[::-1].copy()
    got = download_cache(gpu_append(case, cache=cache, k_bits=k2, v_bits=v2))
    case.k, case.v = W.bf16_bits_to_f32(k2), W.bf16_bits_to_f32(v2)
    assert_cache_equal(got, oracle_cache(case), "overwrite")
