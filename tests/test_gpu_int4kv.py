"""The INT4 cache on the GPU: kv8_quant_append_int4 bit-exact with the
oracle's INT4 quantiser and nibble packing (every bf16 value under fixed
scales, skipped slots, the Llama-3.1-8B-shaped batch), and
paged_decode_attn_int4kv and paged_prefill_chunk_attn_int4kv within
tolerance of the oracle over the same dequantised cache (group sizes, head
dims, q dtypes, split sizes, the full batch over a GPU-written cache,
poisoned slots, single-token exactness; ragged prefill chunks)."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B
from paged_int8_kv_amd import workloads as W
from tests import kv8_testutil as U
from tests.kv8_testutil import (bits_tensor, check_close, dev, f16_to_i16, needs_gpu,
                                oracle_prefill_rows, q_tensor)
from tests.test_gpu_append import assert_cache_equal, rows_case

pytestmark = [pytest.mark.gpu, needs_gpu]


def oracle_cache_int4(case, slots=None):
    kc, vc, ks, vs = O.alloc_paged_cache_int4(case.num_blocks, case.num_kv_heads, case.head_dim)
    O.quant_append_int4(case.k, case.v, case.slot_mapping if slots is None else slots,
                        kc, vc, ks, vs)
    return kc, vc, ks, vs


def upload_int4(kc, vc, ks, vs):
    return (torch.from_numpy(kc).to(dev()), torch.from_numpy(vc).to(dev()),
            torch.from_numpy(f16_to_i16(ks)).to(dev()), torch.from_numpy(f16_to_i16(vs)).to(dev()))


def download(t):
    kc, vc, ks, vs = (x.cpu().numpy() for x in t)
    return kc, vc, ks.view(np.float16), vs.view(np.float16)


def gpu_append_int4(case, slots=None):
    cache = B.alloc_cache(case.num_blocks, case.num_kv_heads, case.head_dim, dev(), int4=True)
    k = bits_tensor(case.k_bits).view(torch.bfloat16)
    v = bits_tensor(case.v_bits).view(torch.bfloat16)
    sl = case.slot_mapping if slots is None else slots
    B.kv8_quant_append_int4(k, v, torch.from_numpy(np.ascontiguousarray(sl, np.int32)).to(dev()),
                            *cache)
    return cache


def gpu_decode_int4(case, cache, tokens_per_split=0, q=None, kernel_form=None):
    qt = q_tensor(case, q)
    b, hq, d = qt.shape
    mcl = int(case.context_lens.max())
    ws = torch.zeros(B.kv8_decode_workspace_size(b, hq, case.num_kv_heads, d, mcl,
                                                 tokens_per_split),
                     dtype=torch.uint8, device=dev())
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=dev())
    B.paged_decode_attn_int4kv(qt, *cache, torch.from_numpy(case.block_table).to(dev()),
                               torch.from_numpy(case.context_lens).to(dev()), mcl, out, ws,
                               tokens_per_split=tokens_per_split,
                               kernel_form=U.form(kernel_form))
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---- append ---------------------------------------------------------------
def test_int4_append_llama8b_bitexact():
    case = W.llama8b_decode(batch=8)
    assert_cache_equal(download(gpu_append_int4(case)), oracle_cache_int4(case), "int4 llama8b")


@pytest.mark.parametrize("absmax", [7.0, 1.0, 0.0234375, 1e-4, 3e-6, 8323072.0, 3.0e38])
def test_int4_append_every_value_for_scale(absmax):
    a = float(W.to_bf16(np.array([absmax], np.float32))[0][0])
    allx = W.bf16_bits_to_f32(np.arange(0x10000, dtype=np.uint32).astype(np.uint16))
    x = allx[np.isfinite(allx) & (np.abs(allx) <= a)]
    d, per = 128, 127
    n = -(-len(x) // per)
    pad = np.zeros(n * per, np.float32)
    pad[:len(x)] = x
    rows = np.concatenate([np.full((n, 1), a, np.float32), pad.reshape(n, per)], axis=1)
    case = rows_case(rows, -rows)
    assert_cache_equal(download(gpu_append_int4(case)), oracle_cache_int4(case),
                       f"int4 values under absmax {absmax}")


def test_int4_append_head_dim_64_and_skipped_slots():
    case = W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=4, head_dim=64,
                             context_lens=[30, 45, 17], k_outliers=True, seed=61)
    slots = case.slot_mapping.copy()
    slots[[0, 7, 44]] = -1
    got = download(gpu_append_int4(case, slots))
    assert_cache_equal(got, oracle_cache_int4(case, slots), "int4 d=64 skipped slots")


# ---- decode ---------------------------------------------------------------
def decode_parity(case, tokens_per_split=0, cache_from="oracle"):
    host = oracle_cache_int4(case)
    if cache_from == "oracle":
        cache = upload_int4(*host)
    else:
        cache = gpu_append_int4(case)
        assert_cache_equal(download(cache), host, "int4 cache written by the GPU")
    out = gpu_decode_int4(case, cache, tokens_per_split)
    ref = O.paged_decode_int4(case.q, *host, case.block_table, case.context_lens)
    check_close(out, ref, f"int4 decode tps={tokens_per_split}")
    return out, host


@pytest.mark.usefixtures("decode_kernel")
@pytest.mark.parametrize("hq,hkv,d,qdt", [
    (4, 4, 128, "bf16"), (8, 4, 64, "f32"), (16, 2, 128, "f32"), (64, 8, 128, "bf16"),
    (8, 1, 64, "bf16"), (32, 8, 128, "f32"),
])
def test_int4_decode_group_sizes_dims_q_dtypes(hq, hkv, d, qdt):
    case = W.make_paged_case(batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             context_lens=[1, 77, 700], q_dtype=qdt, k_outliers=True,
                             seed=hq * 13 + d)
    decode_parity(case)
    decode_parity(case, tokens_per_split=64)


@pytest.mark.usefixtures("decode_kernel")
@pytest.mark.parametrize("tps", [0, 64, 320, 2048])
def test_int4_decode_llama8b_splits(tps):
    decode_parity(W.llama8b_decode(batch=4), tokens_per_split=tps)


@pytest.mark.usefixtures("decode_kernel")
def test_int4_decode_llama8b_full_batch_gpu_cache():
    decode_parity(W.llama8b_decode(), cache_from="gpu")


@pytest.mark.usefixtures("decode_kernel")
def test_int4_decode_single_token_and_poisoned_slots():
    case = W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             context_lens=[1, 23, 40], q_dtype="f32", seed=63, spare_blocks=2)
    kc, vc, ks, vs = oracle_cache_int4(case)
    ref = O.paged_decode_int4(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    used = {(int(case.block_table[b][t // 16]), t % 16)
            for b in range(3) for t in range(int(case.context_lens[b]))}
    for blk in range(case.num_blocks):
        for off in range(16):
            if (blk, off) not in used:
                kc[blk, :, off] = 0x77
                vc[blk, :, off] = 0x99
                ks[blk, :, off] = np.float16(np.inf)
                vs[blk, :, off] = np.float16(np.nan)
    out = gpu_decode_int4(case, upload_int4(kc, vc, ks, vs))
    check_close(out, ref, "int4 poisoned slots")
    v0 = O.gather_dequant_int4(vc, vs, case.block_table[0], 1, 0)[0]
    for h in range(4):
        assert np.array_equal(out[0, h], v0.astype(np.float32))


# ---- prefill --------------------------------------------------------------
def gpu_prefill_int4(case, cache):
    q = bits_tensor(case.q_bits).view(torch.bfloat16)
    qsl = np.ascontiguousarray(case.extra["q_start_loc"], np.int32)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dev())
    B.paged_prefill_chunk_attn_int4kv(
        q, torch.from_numpy(qsl).to(dev()), int(np.max(np.diff(qsl))),
        *cache, torch.from_numpy(case.block_table).to(dev()),
        torch.from_numpy(case.context_lens).to(dev()), int(case.context_lens.max()), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def prefill_parity_int4(case, what, cache_from="oracle"):
    host = oracle_cache_int4(case)
    cache = upload_int4(*host) if cache_from == "oracle" else gpu_append_int4(case)
    out = gpu_prefill_int4(case, cache)
    ref = O.paged_prefill_chunk_int4(case.q, case.extra["q_start_loc"], *host, case.block_table,
                                     case.context_lens)
    check_close(out, ref, what)


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (16, 2, 128), (32, 8, 128), (8, 8, 128)])
def test_int4_prefill_ragged(hq, hkv, d):
    case = W.prefill_case([0, 5, 1000, 17], [1, 77, 300, 0], num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=d, seed=hq * 5 + d + 3, k_outliers=True)
    prefill_parity_int4(case, f"int4 prefill hq={hq} hkv={hkv} d={d}")


def test_int4_prefill_chunked_config_reduced_batch_gpu_cache():
    """The chunked-prefill shape (2 sequences), cache and chunk written by the
    GPU's INT4 append."""
    prefill_parity_int4(W.chunked_prefill(batch=2), "int4 chunked prefill batch 2",
                        cache_from="gpu")


def test_int4_prefill_chunked_config_full_sampled():
    """The full chunked-prefill shape (batch 8) as the benchmark times it:
    cache and chunk written by the GPU's INT4 append, rows sampled across
    every sequence against the oracle over the same cache."""
    case = W.chunked_prefill()
    host = oracle_cache_int4(case)
    cache = gpu_append_int4(case)
    got_cache = [x.cpu().numpy() for x in cache]
    assert np.array_equal(got_cache[0], host[0]) and np.array_equal(got_cache[1], host[1])
    assert np.array_equal(got_cache[2].view(np.float16), host[2])
    assert np.array_equal(got_cache[3].view(np.float16), host[3])
    out = gpu_prefill_int4(case, cache)
    rng = np.random.default_rng(7)
    picks = []
    for b in range(case.batch):
        for i in sorted({0, 1, 63, 64, 255, 256, 511, *rng.integers(0, 512, 3).tolist()}):
            picks.append((b, int(i)))
    ref = oracle_prefill_rows(case, host, picks, gather=O.gather_dequant_int4)
    qsl = case.extra["q_start_loc"]
    got = np.stack([out[qsl[b] + i] for b, i in picks])
    check_close(got, ref, "int4 chunked prefill full, sampled rows")
