"""paged_decode_attn_kv8_append (one decode step: append the newest token of
every sequence, then attend) on the GPU: bitwise equal to kv8_quant_append
followed by paged_decode_attn_kv8 (cache and output), the cache bit-exact
with the oracle's quantiser and the output within tolerance of the oracle,
for new tokens at block and split boundaries, empty and one-token contexts,
several group sizes, head dims, q dtypes and split sizes, and over a
multi-step loop at long context."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B
from paged_int8_kv_amd import workloads as W
from tests import kv8_testutil as U
from tests.kv8_testutil import (bits_tensor, check_close, dev, download_cache, needs_gpu,
                                oracle_cache, q_tensor, upload_cache)
from tests.test_gpu_append import assert_cache_equal

pytestmark = [pytest.mark.gpu, needs_gpu, pytest.mark.usefixtures("decode_kernel")]


def newest_rows(case):
    """Index (into the case's token arrays) of each sequence's newest token,
    or -1 for an empty sequence."""
    idx = np.full(case.batch, -1, np.int64)
    for b in range(case.batch):
        sel = np.nonzero(case.token_seq == b)[0]
        if len(sel):
            idx[b] = sel[np.argmax(case.token_pos[sel])]
    return idx


def cache_before_step(case, idx):
    """The oracle's cache with every newest slot poisoned (as if not yet
    written)."""
    kc, vc, ks, vs = oracle_cache(case)
    for i in idx[idx >= 0]:
        blk, off = divmod(int(case.slot_mapping[i]), 16)
        kc[blk, :, off] = 0x55
        vc[blk, :, off] = -0x55
        ks[blk, :, off] = np.float16(np.nan)
        vs[blk, :, off] = np.float16(np.inf)
    return kc, vc, ks, vs


def new_tokens(case, idx):
    """bf16 bits [B, Hkv, d] of the newest tokens (zeros for empty sequences)."""
    kb = np.zeros((case.batch, case.num_kv_heads, case.head_dim), np.uint16)
    vb = np.zeros_like(kb)
    ok = idx >= 0
    kb[ok] = case.k_bits[idx[ok]]
    vb[ok] = case.v_bits[idx[ok]]
    return bits_tensor(kb).view(torch.bfloat16), bits_tensor(vb).view(torch.bfloat16)


def run_step(case, cache, kn, vn, tps=0, fused=True, block_table=None):
    bt = case.block_table if block_table is None else block_table
    qt = q_tensor(case)
    b, hq, d = qt.shape
    mcl = int(case.context_lens.max())
    ws = torch.zeros(B.kv8_decode_workspace_size(b, hq, case.num_kv_heads, d, mcl, tps),
                     dtype=torch.uint8, device=dev())
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=dev())
    table = torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to(dev())
    lens = torch.from_numpy(case.context_lens).to(dev())
    if fused:
        B.paged_decode_attn_kv8_append(qt, kn, vn, *cache, table, lens, mcl, out, ws,
                                       tokens_per_split=tps, kernel_form=U.form())
    else:
        p = case.context_lens.astype(np.int64) - 1
        slots = np.where(case.context_lens > 0,
                         bt[np.arange(case.batch), np.maximum(p, 0) // 16].astype(np.int64)
                         * 16 + np.maximum(p, 0) % 16, -1)
        slots = np.where((slots < 0) | (slots >= 16 * case.num_blocks), -1, slots).astype(np.int32)
        B.kv8_quant_append(kn, vn, torch.from_numpy(slots).to(dev()), *cache)
        B.paged_decode_attn_kv8(qt, *cache, table, lens, mcl, out, ws, tokens_per_split=tps,
                                kernel_form=U.form())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_step(case, tps=0):
    idx = newest_rows(case)
    before = cache_before_step(case, idx)
    kn, vn = new_tokens(case, idx)
    fused_cache = upload_cache(*before)
    sep_cache = upload_cache(*before)
    out_f = run_step(case, fused_cache, kn, vn, tps, fused=True)
    out_s = run_step(case, sep_cache, kn, vn, tps, fused=False)
    got = download_cache(fused_cache)
    assert_cache_equal(got, download_cache(sep_cache), "fused vs separate cache")
    assert np.array_equal(out_f, out_s), "fused vs separate output"
    full = oracle_cache(case)
    assert_cache_equal(got, full, "fused cache vs oracle")
    ref = O.paged_decode(case.q, *full, case.block_table, case.context_lens)
    check_close(out_f, ref, f"fused step tps={tps}")


def test_fused_step_llama8b_full_batch():
    check_step(W.llama8b_decode())


@pytest.mark.parametrize("tps", [0, 64, 1024])
def test_fused_step_boundaries_and_empty(tps):
    """New tokens at positions 0, 15, 16, 63, 64, 1023, 1024 and in the
    middle of blocks; an empty sequence appends nothing."""
    case = W.make_paged_case(batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[1, 16, 17, 64, 65, 1024, 1025, 0], seed=90 + tps)
    check_step(case, tps)


@pytest.mark.parametrize("hq,hkv,d,qdt", [(8, 2, 64, "f32"), (16, 8, 128, "bf16"),
                                          (64, 8, 128, "bf16"), (4, 4, 64, "f32")])
def test_fused_step_group_sizes(hq, hkv, d, qdt):
    case = W.make_paged_case(batch=5, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             context_lens=[3, 100, 517, 2049, 33], q_dtype=qdt, k_outliers=True,
                             seed=hq + d)
    check_step(case)


def test_fused_steps_long_context_loop():
    """Eight steps of the long-context workload (4 x 32768+ tokens, fp32 q)
    through the fused call; outputs of steps 0 and 7 against the oracle and
    the whole cache bit-exact at the end."""
    case = W.long_context_decode(steps=8)
    cache = upload_cache(*oracle_cache(case))
    kc, vc, ks, vs = oracle_cache(case)
    table = torch.from_numpy(case.block_table).to(dev())
    ws = torch.zeros(B.kv8_decode_workspace_size(4, 32, 8, 128, 32768 + 8), dtype=torch.uint8,
                     device=dev())
    for s in range(8):
        slots = W.step_slots(case, s)
        O.quant_append(case.extra["step_k"][s], case.extra["step_v"][s], slots, kc, vc, ks, vs)
        ctx = (case.context_lens + s + 1).astype(np.int32)
        kn = bits_tensor(case.extra["step_k_bits"][s]).view(torch.bfloat16)
        vn = bits_tensor(case.extra["step_v_bits"][s]).view(torch.bfloat16)
        q = torch.from_numpy(case.extra["step_q"][s].astype(np.float32)).to(dev())
        out = torch.empty((4, 32, 128), dtype=torch.float32, device=dev())
        B.paged_decode_attn_kv8_append(q, kn, vn, *cache, table, torch.from_numpy(ctx).to(dev()),
                                       int(ctx.max()), out, ws, kernel_form=U.form())
        if s in (0, 7):
            ref = O.paged_decode(case.extra["step_q"][s], kc, vc, ks, vs, case.block_table, ctx)
            check_close(out.cpu().numpy(), ref, f"fused long-context step {s}")
    torch.cuda.synchronize()
    assert_cache_equal(download_cache(cache), (kc, vc, ks, vs), "fused loop cache")


def test_fused_step_bad_last_block_id_matches_separate_calls():
    """A last-block id outside [0, num_blocks) (-1, num_blocks, a large
    value): the fused step stores nothing, as kv8_quant_append skips such a
    slot, so cache and output are bitwise those of the two separate calls
    and no other sequence's block is touched."""
    case = W.make_paged_case(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[40, 17, 300, 1], seed=97)
    idx = newest_rows(case)
    before = cache_before_step(case, idx)
    kn, vn = new_tokens(case, idx)
    bt = case.block_table.copy()
    last = (case.context_lens - 1) // 16
    bt[0, last[0]] = -1
    bt[1, last[1]] = case.num_blocks
    bt[2, last[2]] = 1 << 30
    fused_cache = upload_cache(*before)
    sep_cache = upload_cache(*before)
    out_f = run_step(case, fused_cache, kn, vn, fused=True, block_table=bt)
    out_s = run_step(case, sep_cache, kn, vn, fused=False, block_table=bt)
    got = download_cache(fused_cache)
    assert_cache_equal(got, download_cache(sep_cache), "fused vs separate cache, bad ids")
    assert np.array_equal(out_f, out_s), "fused vs separate output, bad ids"
    # only sequence 3's newest slot was written
    exp = [a.copy() for a in before]
    full = oracle_cache(case)
    blk, off = divmod(int(case.slot_mapping[idx[3]]), 16)
    for e, f in zip(exp, full):
        e[blk, :, off] = f[blk, :, off]
    assert_cache_equal(got, tuple(exp), "cache after bad ids")
