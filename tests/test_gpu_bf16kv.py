"""paged_decode_attn_bf16kv (the 16-bit reference point of the equal-memory
comparison) on the GPU against the fp64 oracle over the same bf16 cache:
every supported group size and head dim, both q dtypes, several split
sizes, the Llama-3.1-8B-shaped batch, both item orders, poisoned unused
slots, block permutation (bitwise), single-token exactness and a dominant
key."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B
from paged_int8_kv_amd import workloads as W
from tests.kv8_testutil import bits_tensor, check_close, dev, needs_gpu, q_tensor

pytestmark = [pytest.mark.gpu, needs_gpu]


def upload_bf16(kc, vc):
    return bits_tensor(kc), bits_tensor(vc)


def gpu_decode_bf16(case, cache, q=None, tokens_per_split=0, block_table=None,
                    context_lens=None):
    bt = case.block_table if block_table is None else block_table
    cl = case.context_lens if context_lens is None else context_lens
    mcl = int(np.max(cl))
    qt = q_tensor(case, q)
    b, hq, d = qt.shape
    ws = torch.zeros(B.kv8_decode_workspace_size(b, hq, case.num_kv_heads, d, mcl,
                                                 tokens_per_split),
                     dtype=torch.uint8, device=dev())
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=dev())
    B.paged_decode_attn_bf16kv(qt, *cache,
                               torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to(dev()),
                               torch.from_numpy(np.ascontiguousarray(cl, np.int32)).to(dev()),
                               mcl, out, ws, tokens_per_split=tokens_per_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def parity(case, tokens_per_split=0, what="bf16 kv"):
    kc, vc = W.paged_bf16_cache(case, poison_unused=True)
    out = gpu_decode_bf16(case, upload_bf16(kc, vc), tokens_per_split=tokens_per_split)
    ref = O.paged_decode_bf16(case.q, kc, vc, case.block_table, case.context_lens)
    check_close(out, ref, f"{what} tps={tokens_per_split}")
    return out, ref, (kc, vc)


@pytest.mark.parametrize("hq,hkv,d,qdt", [
    (4, 4, 128, "bf16"), (8, 4, 64, "f32"), (16, 2, 128, "f32"), (64, 8, 128, "bf16"),
    (8, 1, 64, "bf16"), (32, 8, 128, "f32"), (32, 8, 128, "bf16"), (16, 8, 64, "f32"),
])
def test_bf16kv_group_sizes_dims_and_q_dtypes(hq, hkv, d, qdt):
    case = W.make_paged_case(batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             context_lens=[1, 77, 700], q_dtype=qdt, k_outliers=True,
                             seed=hq * 5 + d + (qdt == "f32"), spare_blocks=2)
    parity(case)
    parity(case, tokens_per_split=64)


@pytest.mark.parametrize("tps", [0, 64, 128, 320, 1024, 2048])
def test_bf16kv_llama8b_reduced_batch_splits(tps):
    parity(W.llama8b_decode(batch=4), tokens_per_split=tps)


def test_bf16kv_llama8b_full_batch():
    """The Llama-3.1-8B-shaped batch (32 x 32/8 x 128, contexts 1024..4096,
    bf16 q) over a bf16 cache, default split."""
    parity(W.llama8b_decode())


@pytest.mark.parametrize("batch", [64, 65])
def test_bf16kv_both_item_orders_with_empty_contexts(batch):
    def lens(rng):
        c = rng.integers(0, 700, size=batch)
        c[::9] = 0
        return c
    case = W.make_paged_case(batch=batch, num_q_heads=8, num_kv_heads=2, head_dim=64,
                             context_lens=lens, q_dtype="f32", seed=70 + batch)
    out, _, _ = parity(case, tokens_per_split=128)
    assert np.all(out[case.context_lens == 0] == 0)


def test_bf16kv_single_token_is_its_v():
    case = W.make_paged_case(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             context_lens=[1, 1], q_dtype="f32", seed=75)
    kc, vc = W.paged_bf16_cache(case, poison_unused=True)
    out = gpu_decode_bf16(case, upload_bf16(kc, vc))
    for b in range(2):
        for h in range(8):
            v = O.gather_bf16(vc, case.block_table[b], 1, h // 4)[0]
            assert np.array_equal(out[b, h], v.astype(np.float32))


def test_bf16kv_block_permutation_bitwise():
    base = W.make_paged_case(batch=5, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[3000, 17, 1024, 600, 2500], seed=76, permute=False)
    kc, vc = W.paged_bf16_cache(base)
    out = gpu_decode_bf16(base, upload_bf16(kc, vc))
    perm = np.random.default_rng(3).permutation(base.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    out2 = gpu_decode_bf16(base, upload_bf16(kc2, vc2), block_table=perm[base.block_table])
    assert np.array_equal(out, out2)


def test_bf16kv_dominant_key():
    case = W.make_paged_case(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                             context_lens=[500], q_dtype="f32", seed=77)
    kc, vc = W.paged_bf16_cache(case)
    kd = O.gather_bf16(kc, case.block_table[0], 500, 0)
    q = np.zeros_like(case.q)
    q[0, :] = (kd[123] * (3000.0 / np.dot(kd[123], kd[123]))).astype(np.float32)
    out = gpu_decode_bf16(case, upload_bf16(kc, vc), q=q)
    ref = O.paged_decode_bf16(q, kc, vc, case.block_table, case.context_lens)
    check_close(out, ref, "bf16 kv dominant key")
