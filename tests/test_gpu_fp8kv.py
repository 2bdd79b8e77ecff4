"""The FP8 (e4m3) cache on the GPU: kv8_quant_append_fp8 bit-exact with the
oracle's FP8 quantiser (exhaustive bf16 sweeps, ties, saturation, signed
zero, skipped slots), and paged_decode_attn_fp8kv /
paged_prefill_chunk_attn_fp8kv within tolerance of the oracle over the same
dequantised cache (group sizes, head dims, q dtypes, split sizes, the
Llama-3.1-8B-shaped batch, the chunked-prefill shape, poisoned slots,
single-token exactness)."""
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

pytestmark = [pytest.mark.gpu, needs_gpu, pytest.mark.usefixtures("decode_kernel")]


def oracle_cache_fp8(case):
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, case.num_kv_heads, case.head_dim)
    kc, vc = kc.view(np.uint8), vc.view(np.uint8)
    O.quant_append_fp8(case.k, case.v, case.slot_mapping, kc, vc, ks, vs)
    return kc, vc, ks, vs


def upload_fp8(kc, vc, ks, vs):
    return (torch.from_numpy(kc).to(dev()), torch.from_numpy(vc).to(dev()),
            torch.from_numpy(f16_to_i16(ks)).to(dev()), torch.from_numpy(f16_to_i16(vs)).to(dev()))


def download(t):
    kc, vc, ks, vs = (x.cpu().numpy() for x in t)
    return kc, vc, ks.view(np.float16), vs.view(np.float16)


def gpu_append_fp8(case, cache=None, slots=None):
    if cache is None:
        cache = B.alloc_cache(case.num_blocks, case.num_kv_heads, case.head_dim, dev(), fp8=True)
    k = bits_tensor(case.k_bits).view(torch.bfloat16)
    v = bits_tensor(case.v_bits).view(torch.bfloat16)
    sl = case.slot_mapping if slots is None else slots
    B.kv8_quant_append_fp8(k, v, torch.from_numpy(np.ascontiguousarray(sl, np.int32)).to(dev()),
                           *cache)
    return cache


def gpu_decode_fp8(case, cache, tokens_per_split=0, q=None, kernel_form=None):
    qt = q_tensor(case, q)
    b, hq, d = qt.shape
    mcl = int(case.context_lens.max())
    ws = torch.zeros(B.kv8_decode_workspace_size(b, hq, case.num_kv_heads, d, mcl,
                                                 tokens_per_split),
                     dtype=torch.uint8, device=dev())
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=dev())
    B.paged_decode_attn_fp8kv(qt, *cache, torch.from_numpy(case.block_table).to(dev()),
                              torch.from_numpy(case.context_lens).to(dev()), mcl, out, ws,
                              tokens_per_split=tokens_per_split,
                              kernel_form=U.form(kernel_form))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_prefill_fp8(case, cache):
    q = bits_tensor(case.q_bits).view(torch.bfloat16)
    qsl = np.ascontiguousarray(case.extra["q_start_loc"], np.int32)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dev())
    B.paged_prefill_chunk_attn_fp8kv(
        q, torch.from_numpy(qsl).to(dev()), int(np.max(np.diff(qsl))),
        *cache, torch.from_numpy(case.block_table).to(dev()),
        torch.from_numpy(case.context_lens).to(dev()), int(case.context_lens.max()), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---- append ---------------------------------------------------------------
def test_fp8_append_llama8b_bitexact():
    case = W.llama8b_decode(batch=8)
    assert_cache_equal(download(gpu_append_fp8(case)), oracle_cache_fp8(case), "fp8 llama8b")


@pytest.mark.parametrize("absmax", [448.0, 1.0, 0.0234375, 1e-4, 3e-6, 8323072.0, 3.0e38])
def test_fp8_append_every_value_for_scale(absmax):
    """Every finite bf16 x with |x| <= absmax in rows whose absmax (hence
    scale) is fixed: normal, subnormal, zero and saturated scales; the
    quotients cover every e4m3 code, the subnormal grid, the ties and the
    saturation point."""
    a = float(W.to_bf16(np.array([absmax], np.float32))[0][0])
    allx = W.bf16_bits_to_f32(np.arange(0x10000, dtype=np.uint32).astype(np.uint16))
    x = allx[np.isfinite(allx) & (np.abs(allx) <= a)]
    d, per = 128, 127
    n = -(-len(x) // per)
    pad = np.zeros(n * per, np.float32)
    pad[:len(x)] = x
    rows = np.concatenate([np.full((n, 1), a, np.float32), pad.reshape(n, per)], axis=1)
    case = rows_case(rows, -rows)
    assert_cache_equal(download(gpu_append_fp8(case)), oracle_cache_fp8(case),
                       f"fp8 values under absmax {absmax}")


def test_fp8_append_absmax_sweep_and_signed_zero():
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    a = W.bf16_bits_to_f32(bits)
    rng = np.random.default_rng(31)
    rows = W.to_bf16(rng.uniform(-1, 1, size=(len(a), 64)).astype(np.float32) * a[:, None])[0]
    rows[:, 0] = np.where(np.arange(len(a)) % 2 == 1, -a, a)
    rows[:, 1] = -0.0                                   # negative zero keeps its sign
    case = rows_case(rows, rows[::-1].copy())
    assert_cache_equal(download(gpu_append_fp8(case)), oracle_cache_fp8(case), "fp8 absmax sweep")


def test_fp8_append_skips_negative_slots():
    case = W.make_paged_case(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             context_lens=[30, 45], seed=32)
    slots = case.slot_mapping.copy()
    slots[[0, 7, 44]] = -1
    got = download(gpu_append_fp8(case, slots=slots))
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, 2, 128)
    kc, vc = kc.view(np.uint8), vc.view(np.uint8)
    O.quant_append_fp8(case.k, case.v, slots, kc, vc, ks, vs)
    assert_cache_equal(got, (kc, vc, ks, vs), "fp8 skipped slots")


# ---- decode ---------------------------------------------------------------
def decode_parity(case, tokens_per_split=0, cache_from="oracle"):
    host = oracle_cache_fp8(case)
    if cache_from == "oracle":
        cache = upload_fp8(*host)
    else:
        cache = gpu_append_fp8(case)
        assert_cache_equal(download(cache), host, "fp8 cache written by the GPU")
    out = gpu_decode_fp8(case, cache, tokens_per_split)
    ref = O.paged_decode_fp8(case.q, *host, case.block_table, case.context_lens)
    check_close(out, ref, f"fp8 decode tps={tokens_per_split}")
    return out, host


@pytest.mark.parametrize("hq,hkv,d,qdt", [
    (4, 4, 128, "bf16"), (8, 4, 64, "f32"), (16, 2, 128, "f32"), (64, 8, 128, "bf16"),
    (8, 1, 64, "bf16"), (32, 8, 128, "f32"),
])
def test_fp8_decode_group_sizes_dims_q_dtypes(hq, hkv, d, qdt):
    case = W.make_paged_case(batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             context_lens=[1, 77, 700], q_dtype=qdt, k_outliers=True,
                             seed=hq * 11 + d)
    decode_parity(case)
    decode_parity(case, tokens_per_split=64)


@pytest.mark.parametrize("tps", [0, 64, 320, 2048])
def test_fp8_decode_llama8b_splits(tps):
    decode_parity(W.llama8b_decode(batch=4), tokens_per_split=tps)


def test_fp8_decode_llama8b_full_batch_gpu_cache():
    """The Llama-3.1-8B-shaped batch over an FP8 cache written by the GPU
    append, default split; the cache itself bit-exact too."""
    case = W.llama8b_decode()
    decode_parity(case, cache_from="gpu")


def test_fp8_decode_single_token_and_poisoned_slots():
    case = W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             context_lens=[1, 23, 40], q_dtype="f32", seed=33, spare_blocks=2)
    kc, vc, ks, vs = oracle_cache_fp8(case)
    ref = O.paged_decode_fp8(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    used = {(int(case.block_table[b][t // 16]), t % 16)
            for b in range(3) for t in range(int(case.context_lens[b]))}
    for blk in range(case.num_blocks):
        for off in range(16):
            if (blk, off) not in used:
                kc[blk, :, off] = 0x7E
                vc[blk, :, off] = 0xFE
                ks[blk, :, off] = np.float16(np.inf)
                vs[blk, :, off] = np.float16(np.nan)
    out = gpu_decode_fp8(case, upload_fp8(kc, vc, ks, vs))
    check_close(out, ref, "fp8 poisoned slots")
    v0 = O.gather_dequant_fp8(vc, vs, case.block_table[0], 1, 0)[0]
    for h in range(4):
        assert np.array_equal(out[0, h], v0.astype(np.float32))


# ---- prefill --------------------------------------------------------------
def prefill_parity(case, what):
    host = oracle_cache_fp8(case)
    out = gpu_prefill_fp8(case, upload_fp8(*host))
    ref = O.paged_prefill_chunk_fp8(case.q, case.extra["q_start_loc"], *host, case.block_table,
                                    case.context_lens)
    check_close(out, ref, what)


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (16, 2, 128), (32, 8, 128), (8, 8, 128)])
def test_fp8_prefill_ragged(hq, hkv, d):
    case = W.prefill_case([0, 5, 1000, 17], [1, 77, 300, 0], num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=d, seed=hq * 3 + d + 1, k_outliers=True)
    prefill_parity(case, f"fp8 prefill hq={hq} hkv={hkv} d={d}")


def test_fp8_prefill_chunked_config_reduced_batch():
    prefill_parity(W.chunked_prefill(batch=2), "fp8 chunked prefill batch 2")


def test_fp8_prefill_chunked_config_full_sampled():
    """The full chunked-prefill shape (batch 8) as the benchmark times it:
    cache and chunk written by the GPU's FP8 append (bit-exact with the
    oracle's), rows sampled across every sequence against the oracle."""
    case = W.chunked_prefill()
    host = oracle_cache_fp8(case)
    cache = gpu_append_fp8(case)
    assert_cache_equal(download(cache), host, "fp8 chunked prefill cache")
    out = gpu_prefill_fp8(case, cache)
    rng = np.random.default_rng(7)
    picks = []
    for b in range(case.batch):
        for i in sorted({0, 1, 63, 64, 255, 256, 511, *rng.integers(0, 512, 3).tolist()}):
            picks.append((b, int(i)))
    ref = oracle_prefill_rows(case, host, picks, gather=O.gather_dequant_fp8)
    qsl = case.extra["q_start_loc"]
    got = np.stack([out[qsl[b] + i] for b, i in picks])
    check_close(got, ref, "fp8 chunked prefill full, sampled rows")
