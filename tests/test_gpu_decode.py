"""paged_decode_attn_kv8 on the GPU against the fp64 oracle (same
dequantised cache), plus the invariants the method fixes: block-permutation
invariance (bitwise), single-token exactness, poisoned unused slots, empty
contexts, determinism, any split count."""
import functools

import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B
from paged_int8_kv_amd import workloads as W
from tests import kv8_testutil as U
from tests.kv8_testutil import (check_close, dev, gpu_append, gpu_decode, needs_gpu,
                                oracle_cache, upload_cache)

pytestmark = [pytest.mark.gpu, needs_gpu, pytest.mark.usefixtures("decode_kernel")]


def run_parity(case, tokens_per_split=0, cache_from="oracle"):
    kc, vc, ks, vs = oracle_cache(case)
    cache = upload_cache(kc, vc, ks, vs) if cache_from == "oracle" else gpu_append(case)
    out = gpu_decode(case, cache, tokens_per_split=tokens_per_split)
    ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    return check_close(out, ref, f"decode tps={tokens_per_split}"), out, ref


def test_decode_tiny_config():
    run_parity(W.tiny_decode())


@pytest.mark.parametrize("tps", [0, 64, 128, 320, 512, 2048])
def test_decode_llama8b_reduced_batch_splits(tps):
    run_parity(W.llama8b_decode(batch=4), tokens_per_split=tps)


def test_decode_llama8b_full_batch():
    """Llama-3.1-8B-shaped batch at full size (32 x 32/8 x 128, contexts
    1024..4096), default split as the benchmark launches it, cache built by
    the GPU append kernel."""
    run_parity(W.llama8b_decode(), cache_from="gpu")


@pytest.mark.parametrize("hq,hkv,d,qdt", [
    (4, 4, 128, "bf16"), (8, 4, 64, "f32"), (16, 2, 128, "f32"), (64, 8, 128, "bf16"),
    (8, 1, 64, "bf16"), (32, 8, 128, "f32"),
])
def test_decode_group_sizes_and_dims(hq, hkv, d, qdt):
    case = W.make_paged_case(batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             context_lens=[1, 77, 700], q_dtype=qdt, k_outliers=True,
                             seed=hq * 7 + d)
    run_parity(case)
    run_parity(case, tokens_per_split=64)


def test_decode_long_context_step():
    """Long-context shape (4 x 32768 tokens, 32/8 heads, fp32 q) after one
    appended token per sequence."""
    case = W.long_context_decode(steps=1)
    kc, vc, ks, vs = oracle_cache(case)
    slots = W.step_slots(case, 0)
    O.quant_append(case.extra["step_k"][0], case.extra["step_v"][0], slots, kc, vc, ks, vs)
    ctx = case.context_lens + 1
    cache = upload_cache(kc, vc, ks, vs)
    q = case.extra["step_q"][0]
    out = gpu_decode(case, cache, q=q, context_lens=ctx)
    ref = O.paged_decode(q, kc, vc, ks, vs, case.block_table, ctx)
    check_close(out, ref, "long context")


def test_decode_single_token_is_exact_v():
    case = W.make_paged_case(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[1, 1, 1, 1], seed=31)
    kc, vc, ks, vs = oracle_cache(case)
    out = gpu_decode(case, upload_cache(kc, vc, ks, vs))
    for b in range(4):
        for h in range(32):
            v = O.gather_dequant(vc, vs, case.block_table[b], 1, h // 4)[0]
            assert np.array_equal(out[b, h], v.astype(np.float32))


def test_decode_identical_keys_give_mean_v():
    case = W.make_paged_case(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                             context_lens=[37, 300], seed=32)
    case.k[:] = case.k[0]
    case.k_bits[:] = case.k_bits[0]
    kc, vc, ks, vs = oracle_cache(case)
    out = gpu_decode(case, upload_cache(kc, vc, ks, vs))
    for b in range(2):
        for g in range(2):
            vm = O.gather_dequant(vc, vs, case.block_table[b], int(case.context_lens[b]), g).mean(0)
            for h in range(g * 4, g * 4 + 4):
                check_close(out[b, h], vm, "identical keys")


def test_decode_block_permutation_and_batch_order_bitwise():
    base = W.make_paged_case(batch=5, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[16, 300, 1000, 17, 2048], seed=33, permute=False)
    kc, vc, ks, vs = oracle_cache(base)
    out = gpu_decode(base, upload_cache(kc, vc, ks, vs))
    perm = np.random.default_rng(4).permutation(base.num_blocks)
    arrs = []
    for a in (kc, vc, ks, vs):
        p = np.empty_like(a)
        p[perm] = a
        arrs.append(p)
    out2 = gpu_decode(base, upload_cache(*arrs), block_table=perm[base.block_table])
    assert np.array_equal(out, out2)
    # batch order: the split forms cut each sequence at fixed token offsets,
    # so a reordered batch gives the reordered outputs bit for bit; the
    # stream-K form cuts the whole batch's units into equal ranges, so its
    # pieces (hence roundings) move with the order: within tolerance there
    order = np.array([4, 2, 0, 3, 1])
    out3 = gpu_decode(base, upload_cache(kc, vc, ks, vs), q=base.q_bits[order],
                      block_table=base.block_table[order], context_lens=base.context_lens[order])
    if U.FORM == B.DECODE_STREAMK:
        ref = O.paged_decode(base.q, kc, vc, ks, vs, base.block_table, base.context_lens)
        check_close(out3, ref[order], "stream-K reordered batch")
    else:
        assert np.array_equal(out3, out[order])


def test_decode_poisoned_unused_slots_and_empty_context():
    case = W.make_paged_case(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128,
                             context_lens=[21, 0, 70], seed=34, spare_blocks=3)
    kc, vc, ks, vs = oracle_cache(case)
    ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    # poison every slot beyond each context and the spare blocks
    used = set()
    for b in range(3):
        n = int(case.context_lens[b])
        for t in range(n):
            used.add((int(case.block_table[b][t // 16]), t % 16))
    nanbits = np.float16(np.nan)
    for blk in range(case.num_blocks):
        for off in range(16):
            if (blk, off) not in used:
                kc[blk, :, off] = 127
                vc[blk, :, off] = -127
                ks[blk, :, off] = nanbits
                vs[blk, :, off] = np.float16(np.inf)
    out = gpu_decode(case, upload_cache(kc, vc, ks, vs))
    assert np.all(out[1] == 0)
    check_close(out, ref, "poisoned")


def test_decode_deterministic_and_context_cap():
    case = W.llama8b_decode(batch=6)
    kc, vc, ks, vs = oracle_cache(case)
    cache = upload_cache(kc, vc, ks, vs)
    a = gpu_decode(case, cache)
    b = gpu_decode(case, cache)
    assert np.array_equal(a, b)
    # max_context_len below some lengths clamps those sequences
    cap = 2000
    out = gpu_decode(case, cache, max_context_len=cap)
    ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table,
                         np.minimum(case.context_lens, cap))
    check_close(out, ref, "context cap")


def test_decode_large_logits_dominant_key():
    case = W.make_paged_case(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                             context_lens=[500], q_dtype="f32", seed=35)
    kc, vc, ks, vs = oracle_cache(case)
    kd = O.gather_dequant(kc, ks, case.block_table[0], 500, 0)
    q = np.zeros_like(case.q)
    q[0, :] = (kd[123] * (3000.0 / np.dot(kd[123], kd[123]))).astype(np.float32)
    out = gpu_decode(case, upload_cache(kc, vc, ks, vs), q=q)
    ref = O.paged_decode(q, kc, vc, ks, vs, case.block_table, case.context_lens)
    check_close(out, ref, "dominant key")


def test_decode_workspace_reused_across_calls():
    """One zero-filled workspace serves many calls of different shapes: the
    split counters return to zero after every call."""
    big = W.llama8b_decode(batch=8)
    small = W.make_paged_case(batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
                              context_lens=[5000, 64, 1500], seed=36)
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device=dev())
    for case in (big, small, big, small):
        kc, vc, ks, vs = oracle_cache(case)
        for tps in (64, 256):
            out = gpu_decode(case, upload_cache(kc, vc, ks, vs), tokens_per_split=tps,
                             workspace=ws)
            ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
            check_close(out, ref, f"reused workspace tps={tps}")
    assert int(ws[:4 * B.MAX_DECODE_PAIRS].count_nonzero()) == 0   # counters back to zero


def test_decode_workspace_reused_across_pair_counts():
    """One zero-filled workspace reused while batch * Hkv crosses a
    64-counter boundary both ways (8x8 -> 32x8 -> 3x8 -> 32x8 pairs): the
    counters live at fixed positions ahead of every partial, so no call
    reads a counter another call's partials overwrote; every output element
    is written (NaN-filled beforehand) and within tolerance."""
    def case_of(batch, seed):
        rng = np.random.default_rng(seed)
        return W.make_paged_case(batch=batch, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                 context_lens=list(rng.integers(300, 2500, batch)), seed=seed)
    cases = [case_of(8, 70), case_of(32, 71), case_of(3, 72), case_of(32, 73)]
    ws = torch.zeros(max(B.kv8_decode_workspace_size(c.batch, 32, 8, 128,
                                                     int(c.context_lens.max()), 128)
                         for c in cases), dtype=torch.uint8, device=dev())
    for c in cases:
        kc, vc, ks, vs = oracle_cache(c)
        out = gpu_decode(c, upload_cache(kc, vc, ks, vs), tokens_per_split=128, workspace=ws)
        ref = O.paged_decode(c.q, kc, vc, ks, vs, c.block_table, c.context_lens)
        check_close(out, ref, f"reused workspace, {c.batch} sequences")
    assert int(ws[:4 * B.MAX_DECODE_PAIRS].count_nonzero()) == 0


@functools.lru_cache(maxsize=None)
def max_pairs_case():
    """4096 sequences x 16 KV heads, contexts of 0..40 tokens (every 97th
    empty), with its oracle cache and output, built once and shared by the
    kernel forms."""
    def lens(rng):
        c = rng.integers(0, 41, size=4096)
        c[::97] = 0
        return c
    case = W.make_paged_case(batch=4096, num_q_heads=64, num_kv_heads=16, head_dim=64,
                             context_lens=lens, seed=130)
    kc, vc, ks, vs = oracle_cache(case)
    ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    return case, (kc, vc, ks, vs), ref


def test_decode_max_pairs():
    """The most (sequence, KV head) pairs one call takes: 4096 x 16 = 65536,
    KV8_DECODE_MAX_PAIRS.  The split counters fill the fixed counter region
    to its last word (stream-K's one word apart), and the items keep
    sequence order (more than 64 sequences).  Every output element is
    written (NaN-filled beforehand) and within tolerance of the oracle, the
    empty contexts give exact zeros, and the counters are left zero."""
    case, oc, ref = max_pairs_case()
    assert case.batch * case.num_kv_heads == B.MAX_DECODE_PAIRS
    ws = torch.zeros(B.kv8_decode_workspace_size(case.batch, 64, 16, 64,
                                                 int(case.context_lens.max()), 0),
                     dtype=torch.uint8, device=dev())
    out = gpu_decode(case, upload_cache(*oc), workspace=ws)
    check_close(out, ref, "65536 pairs")
    assert np.all(out[case.context_lens == 0] == 0.0)
    assert int(ws[:4 * B.MAX_DECODE_PAIRS].count_nonzero()) == 0


@pytest.mark.parametrize("tps", [0, 128, 1024])
def test_decode_rising_logits_rescale_every_block(tps):
    """Keys whose logits climb block after block (about 9 in log2 units per
    16 tokens) move every wave's running max on every block, so the
    accumulator rescale runs each time; also contexts of 1 block, a few
    blocks and many blocks per wave."""
    for ctx in ([5], [200], [3000]):
        case = W.make_paged_case(batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                 context_lens=ctx, q_dtype="f32", seed=50 + ctx[0])
        n = int(case.context_lens[0])
        u = np.zeros(128, np.float32)
        u[:8] = 1.0
        ramp = (np.arange(n, dtype=np.float32) / 16.0) * 1.5     # ~9 log2 units per block
        k = case.k.copy()
        k[:, :, :8] = ramp[:, None, None] + 0.05 * k[:, :, :8]
        case.k, case.k_bits = W.to_bf16(k)
        case.q[:] = 0.0
        case.q[:, :, :8] = 6.0
        kc, vc, ks, vs = oracle_cache(case)
        out = gpu_decode(case, upload_cache(kc, vc, ks, vs), tokens_per_split=tps)
        ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
        check_close(out, ref, f"rising logits ctx={ctx} tps={tps}")


@pytest.mark.parametrize("batch", [64, 65, 97])
def test_decode_many_sequences_both_item_orders(batch):
    """Up to 64 sequences the work items are ranked longest first; above
    that they keep sequence order.  Both orders, with ragged contexts
    (empty ones included) and a split size that gives several splits of
    unequal block counts, match the oracle."""
    def lens(rng):
        c = rng.integers(0, 700, size=batch)
        c[::9] = 0
        c[1::13] = 16 * rng.integers(1, 40, size=c[1::13].shape)
        return c
    case = W.make_paged_case(batch=batch, num_q_heads=8, num_kv_heads=2, head_dim=64,
                             context_lens=lens, seed=60 + batch)
    run_parity(case)
    run_parity(case, tokens_per_split=128)


@functools.lru_cache(maxsize=None)
def constant_sign_case(hq, hkv, logits):
    """The adversarial case below with its oracle cache and output, built
    once per shape and shared by the kernel forms."""
    case = W.make_paged_case(batch=4, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                             context_lens=[32768, 20000, 2049, 4097], q_dtype="f32",
                             seed=80 + hq)
    rng = np.random.default_rng(81 + hq)
    sign = np.where(rng.random((hkv, 128)) < 0.5, -1.0, 1.0).astype(np.float32)
    mag = rng.uniform(0.5, 4.0, size=(case.k.shape[0], 1, 1)).astype(np.float32)
    v = sign[None] * mag * (1.0 - 0.02 * rng.random(case.v.shape, dtype=np.float32))
    case.v, case.v_bits = W.to_bf16(v)
    if logits == "flat":
        case.q[:] = 0.0
    else:
        case.q *= np.float32(0.004)
    cache = oracle_cache(case)
    ref = O.paged_decode(case.q, *cache, case.block_table, case.context_lens)
    return case, cache, ref


@pytest.mark.parametrize("logits", ["flat", "near_flat"])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8)])
def test_decode_adversarial_long_splits_constant_sign_values(hq, hkv, logits):
    """Accumulator headroom.  Every V element of a head keeps one sign over
    all tokens and sits within 2% of the token's absmax, so the INT8 codes
    are all near +-127 of one sign and nothing cancels; Q is zero (every
    logit 0, every weight equal) or tiny (logits within about +-0.05).  Each
    split then sums its weighted codes to roughly split_len * 127 before the
    merge, the largest sums the kernels ever hold.  Splits of 2048 tokens
    (1280 at G = 8 for the forms that keep a split's logits in LDS), a
    32768-token sequence beside shorter ragged ones."""
    G = hq // hkv
    tps = 1280 if G == 8 and U.FORM in (B.DECODE_DOT, B.DECODE_MFMA) else 2048
    case, (kc, vc, ks, vs), ref = constant_sign_case(hq, hkv, logits)
    codes = vc.astype(np.int32)
    assert np.abs(codes[codes != 0]).min() >= 120
    out = gpu_decode(case, upload_cache(kc, vc, ks, vs), tokens_per_split=tps)
    check_close(out, ref, f"constant-sign V, {logits} logits, G={G}, tps={tps}")
