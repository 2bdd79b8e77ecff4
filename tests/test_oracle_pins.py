"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

CPU only.  None of these re-types the oracle's own formula: the quantiser is
checked against exact rational / exact-residual rounding, attention against
brute force on tiny inputs, against torch's scaled_dot_product_attention in
fp64 (the dense, non-paged, MHA special case), against closed forms
(single token, identical keys) and against invariants (block permutation,
batch order, causal locality).  The KV-size closed form reproduces the
numbers the overview page ("KV Cache 优化全景解析") prints.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers independent of the oracle
# ---------------------------------------------------------------------------
def all_finite_bf16(positive_only=False):
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = W.bf16_bits_to_f32(bits)
    keep = np.isfinite(vals)
    if positive_only:
        keep &= vals > 0
    return vals[keep]


def fp16_rne_exact(r):
    """Round a non-negative rational to fp16 (nearest even, subnormals),
    returning math.inf on overflow.  Pure integer/rational arithmetic."""
    if r == 0:
        return 0.0
    e = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    quantum = Fraction(2) ** (max(e, -14) - 10)
    k = round(r / quantum)          # Fraction.__round__ rounds half to even
    val = k * quantum
    if val > 65504:
        return math.inf
    return float(val)


def exact_codes(x, s):
    """round_half_even(x / s) clamped to +-127, decided by an exact residual
    test in fp64 (every product and difference below is exact)."""
    x = np.asarray(x, np.float64)
    s = float(s)
    if s == 0:
        return np.zeros(x.shape, np.int64)
    big = np.abs(x) > 200 * s
    xs = np.where(big, 0.0, x)
    k = np.floor(xs / s)
    r = xs - k * s
    k = np.where(r < 0, k - 1, k)
    r = xs - k * s
    k = np.where(r >= s, k + 1, k)
    r = xs - k * s
    up = (2 * r > s) | ((2 * r == s) & (np.mod(k, 2) == 1))
    c = k + up
    c = np.where(big, np.sign(x) * 127, c)
    return np.clip(c, -127, 127).astype(np.int64)


def quantize_reference_rows(rows):
    """Quantise rows with the exact helpers above (scale from Fraction)."""
    codes, scales = [], []
    for row in rows:
        a = max(abs(float(v)) for v in row)
        s = fp16_rne_exact(Fraction(a) / 127)
        if s == math.inf:
            s = 65504.0
        codes.append(exact_codes(row, s))
        scales.append(s)
    return np.array(codes), np.array(scales)


def brute_attention(q, k, v, scale):
    """Dense softmax attention of one query over rows of k/v, pure python."""
    logits = [scale * sum(float(a) * float(b) for a, b in zip(q, kr)) for kr in k]
    m = max(logits)
    w = [math.exp(z - m) for z in logits]
    tot = sum(w)
    return [sum(wi * float(vr[i]) for wi, vr in zip(w, v)) / tot for i in range(len(q))]


def build_cache(case):
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, case.num_kv_heads, case.head_dim)
    O.quant_append(case.k, case.v, case.slot_mapping, kc, vc, ks, vs)
    return kc, vc, ks, vs


def dense_dequant(case, b, which):
    """Contiguous dequantised [ctx, Hkv, d] of sequence b, quantised from the
    source tokens in sequence order (no block table involved)."""
    src = case.k if which == "k" else case.v
    rows = src[case.token_seq == b]
    codes, scales = O.quantize_rows(rows)
    return O.dequantize_rows(codes, scales)


# ---------------------------------------------------------------------------
# KV-size closed form ("KV Cache 优化全景解析", sections 2.3 / 3.3 / 11.4)
# ---------------------------------------------------------------------------
def test_kv_size_printed_tables():
    g = json.load(open(os.path.join(GOLDEN, "kv_size_tables.json")))
    t = g["llama3_70b_fp16_by_length"]
    for seq, printed in t["rows"]:
        gib = O.kv_cache_bytes(t["num_layers"], t["batch"], seq, t["num_kv_heads"],
                               t["head_dim"], t["bytes"]) / 1024 ** 3
        assert f"{gib:.2f}" == printed
    t = g["llama3_70b_8k_by_attention_type"]
    for _, heads, printed in t["rows"]:
        gib = O.kv_cache_bytes(t["num_layers"], t["batch"], t["seq_len"], heads,
                               t["head_dim"], t["bytes"]) / 1024 ** 3
        assert f"{gib:.2f}" == printed
    t = g["llama3_8b_b16_t8k"]
    for _, nbytes, printed in t["rows"]:
        gib = O.kv_cache_bytes(t["num_layers"], t["batch"], t["seq_len"], t["num_kv_heads"],
                               t["head_dim"], nbytes) / 1024 ** 3
        assert f"{gib:.2f}" == printed


@pytest.mark.parametrize("layers,batch,tokens,hkv,d", [(1, 1, 256, 1, 64), (2, 3, 4096, 8, 128)])
def test_paged_allocation_matches_closed_form(layers, batch, tokens, hkv, d):
    nb = batch * tokens // O.BLOCK_SIZE
    arrays = O.alloc_paged_cache(nb, hkv, d)
    code_bytes = layers * (arrays[0].nbytes + arrays[1].nbytes)
    assert code_bytes == O.kv_cache_bytes(layers, batch, tokens, hkv, d, 1)
    scale_bytes = layers * (arrays[2].nbytes + arrays[3].nbytes)
    assert scale_bytes == O.kv_cache_bytes(layers, batch, tokens, hkv, 1, 2)
    assert layers * O.paged_cache_bytes(nb, hkv, d) == code_bytes + scale_bytes


# ---------------------------------------------------------------------------
# Quantiser
# ---------------------------------------------------------------------------
def test_scale_exhaustive_all_bf16_absmax():
    a = all_finite_bf16(positive_only=True)
    got = O.row_scale(a[:, None]).astype(np.float64)
    exp = []
    for v in a.tolist():
        s = fp16_rne_exact(Fraction(v) / 127)
        exp.append(65504.0 if s == math.inf else s)
    exp = np.array(exp)
    assert np.array_equal(got, exp)
    # the fp64-quotient reading gives the same scales on the whole bf16 domain
    with np.errstate(over="ignore"):
        s64 = (a.astype(np.float64) / 127.0).astype(np.float16)
    s64 = np.where(np.isinf(s64), np.float16(65504), s64).astype(np.float64)
    assert np.array_equal(got, s64)


def test_scale_edges():
    # smallest absmax whose scale is non-zero, saturation threshold
    assert O.row_scale(np.array([[0.0, 0.0]]))[0] == 0
    assert O.row_scale(np.array([[3.78e-6]]).astype(np.float32))[0] == 0
    assert O.row_scale(np.array([[8257536.0]]))[0] == np.float16(65024)
    assert O.row_scale(np.array([[8323072.0]]))[0] == np.float16(65504)


# 14 and 0.875: scales whose fp32 reciprocal is inexact, where x * fp32(1/s)
# rounds 6 bf16 values differently from the specified division
SCALES = [1.0, 0.0234375, 0.5 + 2 ** -11, 6.103515625e-05, 2 ** -24, 3 * 2 ** -24,
          1000 * 2 ** -24, 65504.0, 2.0 ** 10 * 1.5, 14.0, 0.875]


@pytest.mark.parametrize("s", SCALES)
def test_codes_exhaustive_all_bf16(s):
    x = all_finite_bf16()
    got = O.codes_for_scale(x[None, :], np.array([s], np.float16))[0].astype(np.int64)
    assert np.array_equal(got, exact_codes(x, np.float16(s)))


def test_codes_fraction_spot_check():
    rng = np.random.default_rng(11)
    x = all_finite_bf16()
    pick = x[rng.choice(len(x), 3000, replace=False)]
    for s in (0.0234375, 3 * 2 ** -24, 1.0):
        got = O.codes_for_scale(pick[None, :], np.array([s], np.float16))[0]
        for xv, c in zip(pick.tolist(), got.tolist()):
            q = round(Fraction(xv) / Fraction(s))
            assert c == max(-127, min(127, q))


def test_quantize_rows_random_vs_exact():
    rng = np.random.default_rng(5)
    rows, _ = W.to_bf16(rng.standard_normal((300, 64)).astype(np.float32)
                        * np.exp(rng.uniform(-18, 18, size=(300, 1))).astype(np.float32))
    codes, scales = O.quantize_rows(rows)
    rc, rs = quantize_reference_rows(rows)
    assert np.array_equal(scales.astype(np.float64), rs)
    assert np.array_equal(codes.astype(np.int64), rc)


def test_quantiser_invariants():
    rng = np.random.default_rng(7)
    rows, _ = W.to_bf16(rng.standard_normal((500, 128)).astype(np.float32))
    c, s = O.quantize_rows(rows)
    cn, sn = O.quantize_rows(-rows)
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    for k in (-3, 5):
        c2, s2 = O.quantize_rows(rows * 2.0 ** k)
        assert np.array_equal(c2, c)
        assert np.array_equal(s2.astype(np.float64), s.astype(np.float64) * 2.0 ** k)
    err = np.abs(rows - O.dequantize_rows(c, s))
    assert np.all(err <= s.astype(np.float64)[:, None] / 2)
    am = np.argmax(np.abs(rows), axis=1)
    assert np.all(np.abs(c[np.arange(500), am]) == 127)
    assert c.min() >= -127


def test_quantiser_ties_to_even_and_clamp():
    row = np.array([[127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -1.5]])
    c, s = O.quantize_rows(row)
    assert s[0] == 1.0
    assert c[0].tolist() == [127, 2, 4, -2, 0, 0, 2, -2]
    # subnormal scale: the absmax element's quotient exceeds 127 -> clamped
    row = np.array([[np.float32(1e-4), -np.float32(1e-4)]]).astype(np.float64)
    row = W.to_bf16(row.astype(np.float32))[0]
    c, s = O.quantize_rows(row)
    assert 0 < s[0] < np.float16(6.103515625e-05)
    assert c[0].tolist() == [127, -127]
    assert row[0, 0] / float(s[0]) > 127.5


# ---------------------------------------------------------------------------
# Append (scatter through slot mapping)
# ---------------------------------------------------------------------------
def test_append_scatter_and_skip():
    case = W.make_paged_case(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=16,
                             context_lens=[21, 40], seed=9)
    slots = case.slot_mapping.copy()
    slots[3] = -1
    # one spare block past the pool, never a slot's target: a skipped row
    # written anyway (e.g. at slot -1, the last slot of the last block)
    # lands there and shows
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks + 1, 2, 16)
    O.quant_append(case.k, case.v, slots, kc, vc, ks, vs)
    codes_k, sc_k = quantize_reference_rows(case.k.reshape(-1, 16))
    codes_k = codes_k.reshape(case.k.shape)
    sc_k = sc_k.reshape(case.k.shape[:2])
    exp_kc = np.zeros(kc.shape, np.int64)
    exp_ks = np.zeros(ks.shape, np.float64)
    for n in range(len(slots)):
        blk, off = divmod(int(case.slot_mapping[n]), 16)
        if n == 3:
            assert np.all(kc[blk, :, off] == 0) and np.all(ks[blk, :, off] == 0)
            continue
        assert np.array_equal(kc[blk, :, off].astype(np.int64), codes_k[n])
        assert np.array_equal(ks[blk, :, off].astype(np.float64), sc_k[n])
        exp_kc[blk, :, off] = codes_k[n]
        exp_ks[blk, :, off] = sc_k[n]
    # nothing is written anywhere else: not the skipped row under any other
    # reading of its slot, not the blocks' unused tails
    assert np.array_equal(kc.astype(np.int64), exp_kc)
    assert np.array_equal(ks.astype(np.float64), exp_ks)
    written = np.zeros(vs.shape, bool)
    for n in range(len(slots)):
        if n != 3:
            blk, off = divmod(int(case.slot_mapping[n]), 16)
            written[blk, :, off] = True
    assert np.all(vc[~written] == 0) and np.all(vs[~written] == 0)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def test_decode_brute_force_tiny():
    case = W.make_paged_case(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8,
                             context_lens=[5, 37], q_dtype="f32", seed=3)
    kc, vc, ks, vs = build_cache(case)
    out = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    for b in range(2):
        K = dense_dequant(case, b, "k")
        V = dense_dequant(case, b, "v")
        for h in range(4):
            g = h // 2
            ref = brute_attention(case.q[b, h], K[:, g], V[:, g], 1 / math.sqrt(8))
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)


def sdpa_decode(case, kc, vc, ks, vs):
    outs = []
    for b in range(case.batch):
        ctx = int(case.context_lens[b])
        K = np.stack([O.gather_dequant(kc, ks, case.block_table[b], ctx, g)
                      for g in range(case.num_kv_heads)])
        V = np.stack([O.gather_dequant(vc, vs, case.block_table[b], ctx, g)
                      for g in range(case.num_kv_heads)])
        Kt = torch.from_numpy(K).repeat_interleave(case.group, dim=0)[None]
        Vt = torch.from_numpy(V).repeat_interleave(case.group, dim=0)[None]
        q = torch.from_numpy(case.q[b].astype(np.float64))[None, :, None, :]
        outs.append(torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt)[0, :, 0].numpy())
    return np.stack(outs)


@pytest.mark.parametrize("maker", [
    lambda: W.tiny_decode(),
    lambda: W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=32,
                              context_lens=[1, 17, 300], q_dtype="bf16", k_outliers=True, seed=4),
    lambda: W.make_paged_case(batch=2, num_q_heads=4, num_kv_heads=4, head_dim=16,
                              context_lens=[33, 64], seed=5),       # MHA, G = 1
    lambda: W.make_paged_case(batch=2, num_q_heads=6, num_kv_heads=1, head_dim=16,
                              context_lens=[48, 7], seed=6),        # MQA, Hkv = 1
])
def test_decode_matches_sdpa_fp64(maker):
    case = maker()
    kc, vc, ks, vs = build_cache(case)
    out = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    ref = sdpa_decode(case, kc, vc, ks, vs)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_decode_closed_forms():
    case = W.make_paged_case(batch=3, num_q_heads=4, num_kv_heads=1, head_dim=16,
                             context_lens=[1, 20, 0], seed=8)
    kc, vc, ks, vs = build_cache(case)
    out = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    # single token: exactly its dequantised V
    v0 = O.gather_dequant(vc, vs, case.block_table[0], 1, 0)[0]
    for h in range(4):
        assert np.array_equal(out[0, h], v0)
    # empty context: zeros
    assert np.all(out[2] == 0)
    # identical keys: mean of dequantised V; and q = 0 gives the same
    blk = case.block_table[1]
    for t in range(20):
        b_, o_ = blk[t // 16], t % 16
        kc[b_, 0, o_] = kc[blk[0], 0, 0]
        ks[b_, 0, o_] = ks[blk[0], 0, 0]
    out = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    vmean = O.gather_dequant(vc, vs, blk, 20, 0).mean(axis=0)
    assert np.allclose(out[1], vmean[None, :], rtol=1e-13, atol=1e-14)
    q0 = np.zeros_like(case.q)
    out0 = O.paged_decode(q0, kc, vc, ks, vs, case.block_table, case.context_lens)
    assert np.allclose(out0[1], vmean[None, :], rtol=1e-13, atol=1e-14)


def test_decode_dominant_key_large_logits():
    # logits near 1e3: the max-subtracted softmax must still return the
    # dominant token's V (an unstabilised exp overflows)
    case = W.make_paged_case(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=16,
                             context_lens=[40], q_dtype="f32", seed=12)
    kc, vc, ks, vs = build_cache(case)
    t_star = 23
    blk, off = case.block_table[0][t_star // 16], t_star % 16
    kd = O.gather_dequant(kc, ks, case.block_table[0], 40, 0)
    q = np.zeros_like(case.q)
    q[0, :] = kd[t_star] * (4000.0 / np.dot(kd[t_star], kd[t_star]))
    out = O.paged_decode(q, kc, vc, ks, vs, case.block_table, case.context_lens)
    v_star = O.dequantize_rows(vc[blk, 0, off][None], vs[blk, 0, off][None])[0]
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0, 0], v_star, atol=1e-6)


def test_block_permutation_and_batch_shuffle_invariance():
    base = W.make_paged_case(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                             context_lens=[50, 3, 97], seed=10, permute=False)
    kc, vc, ks, vs = build_cache(base)
    ref = O.paged_decode(base.q, kc, vc, ks, vs, base.block_table, base.context_lens)
    rng = np.random.default_rng(1)
    perm = rng.permutation(base.num_blocks)        # physical block p -> perm[p]
    kc2, vc2, ks2, vs2 = (np.empty_like(a) for a in (kc, vc, ks, vs))
    for src, dst in ((kc, kc2), (vc, vc2), (ks, ks2), (vs, vs2)):
        dst[perm] = src
    table2 = perm[base.block_table]
    out = O.paged_decode(base.q, kc2, vc2, ks2, vs2, table2, base.context_lens)
    assert np.array_equal(out, ref)
    order = np.array([2, 0, 1])
    out = O.paged_decode(base.q[order], kc, vc, ks, vs, base.block_table[order],
                         base.context_lens[order])
    assert np.array_equal(out, ref[order])


def test_block_table_example_from_page():
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    phys = g["request_a"]["physical"]
    rng = np.random.default_rng(2)
    rows, _ = W.to_bf16(rng.standard_normal((48, 1, 8)).astype(np.float32))
    kc, vc, ks, vs = O.alloc_paged_cache(10, 1, 8)
    slots = [phys[t // 16] * 16 + t % 16 for t in range(48)]
    O.quant_append(rows, rows, slots, kc, vc, ks, vs)
    # the free pool's blocks stay untouched
    for p in g["free_pool_prefix"]:
        assert np.all(kc[p] == 0)
    got = O.gather_dequant(kc, ks, np.array(phys), 48, 0)
    c, s = O.quantize_rows(rows[:, 0])
    assert np.array_equal(got, O.dequantize_rows(c, s))


# ---------------------------------------------------------------------------
# Chunked prefill
# ---------------------------------------------------------------------------
def test_prefill_no_context_equals_sdpa_causal():
    case = W.chunked_prefill(seed=21, batch=2, chunk=24, lo=0, hi=0,
                             num_q_heads=4, num_kv_heads=2, head_dim=16)
    kc, vc, ks, vs = build_cache(case)
    qsl = case.extra["q_start_loc"]
    out = O.paged_prefill_chunk(case.q, qsl, kc, vc, ks, vs, case.block_table, case.context_lens)
    for b in range(2):
        K = np.stack([O.gather_dequant(kc, ks, case.block_table[b], 24, g) for g in range(2)])
        V = np.stack([O.gather_dequant(vc, vs, case.block_table[b], 24, g) for g in range(2)])
        Kt = torch.from_numpy(K).repeat_interleave(2, dim=0)[None]
        Vt = torch.from_numpy(V).repeat_interleave(2, dim=0)[None]
        q = torch.from_numpy(case.q[qsl[b]:qsl[b + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, is_causal=True)
        assert np.allclose(out[qsl[b]:qsl[b + 1]], ref[0].permute(1, 0, 2).numpy(),
                           rtol=1e-11, atol=1e-12)


def test_prefill_with_context_equals_sdpa_masked_and_locality():
    case = W.chunked_prefill(seed=22, batch=2, chunk=9, lo=20, hi=40,
                             num_q_heads=4, num_kv_heads=1, head_dim=16)
    kc, vc, ks, vs = build_cache(case)
    qsl = case.extra["q_start_loc"]
    out = O.paged_prefill_chunk(case.q, qsl, kc, vc, ks, vs, case.block_table, case.context_lens)
    for b in range(2):
        ctx = int(case.context_lens[b])
        prev = ctx - 9
        K = O.gather_dequant(kc, ks, case.block_table[b], ctx, 0)
        V = O.gather_dequant(vc, vs, case.block_table[b], ctx, 0)
        mask = np.arange(ctx)[None, :] <= (prev + np.arange(9))[:, None]
        q = torch.from_numpy(case.q[qsl[b]:qsl[b + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
            attn_mask=torch.from_numpy(mask))
        assert np.allclose(out[qsl[b]:qsl[b + 1]], ref[0].permute(1, 0, 2).numpy(),
                           rtol=1e-11, atol=1e-12)
    # causal locality: changing the last token's K/V leaves earlier rows alone
    b = 1
    ctx = int(case.context_lens[b])
    t = ctx - 1
    blk, off = case.block_table[b][t // 16], t % 16
    kc[blk, 0, off] = -kc[blk, 0, off]
    vc[blk, 0, off] = 127
    out2 = O.paged_prefill_chunk(case.q, qsl, kc, vc, ks, vs, case.block_table, case.context_lens)
    r1 = qsl[b + 1]
    assert np.array_equal(out2[:r1 - 1], out[:r1 - 1])
    assert not np.allclose(out2[r1 - 1], out[r1 - 1])


def test_prefill_single_row_equals_decode():
    case = W.chunked_prefill(seed=23, batch=3, chunk=1, lo=5, hi=70,
                             num_q_heads=8, num_kv_heads=2, head_dim=32)
    kc, vc, ks, vs = build_cache(case)
    out_p = O.paged_prefill_chunk(case.q, case.extra["q_start_loc"], kc, vc, ks, vs,
                                  case.block_table, case.context_lens)
    out_d = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    assert np.allclose(out_p, out_d, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# 16-bit KV reference point (README section 实验效果: KV8 against FA2 over the
# unquantised cache)
# ---------------------------------------------------------------------------
def dense_bf16(case, b):
    """Contiguous [ctx, Hkv, d] source rows of sequence b in sequence order
    (no block table involved)."""
    return case.k[case.token_seq == b].astype(np.float64), case.v[case.token_seq == b].astype(np.float64)


def test_bf16_decode_brute_force_tiny():
    case = W.make_paged_case(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8,
                             context_lens=[5, 37], q_dtype="f32", seed=13)
    kc, vc = W.paged_bf16_cache(case, poison_unused=True)
    out = O.paged_decode_bf16(case.q, kc, vc, case.block_table, case.context_lens)
    for b in range(2):
        K, V = dense_bf16(case, b)
        for h in range(4):
            ref = brute_attention(case.q[b, h], K[:, h // 2], V[:, h // 2], 1 / math.sqrt(8))
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)


def test_bf16_decode_matches_sdpa_fp64():
    case = W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=32,
                             context_lens=[1, 17, 300], q_dtype="bf16", k_outliers=True, seed=14)
    kc, vc = W.paged_bf16_cache(case)
    out = O.paged_decode_bf16(case.q, kc, vc, case.block_table, case.context_lens)
    for b in range(3):
        K, V = dense_bf16(case, b)
        Kt = torch.from_numpy(K.transpose(1, 0, 2)).repeat_interleave(4, dim=0)[None]
        Vt = torch.from_numpy(V.transpose(1, 0, 2)).repeat_interleave(4, dim=0)[None]
        q = torch.from_numpy(case.q[b].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt)[0, :, 0].numpy()
        assert np.allclose(out[b], ref, rtol=1e-11, atol=1e-12)


def test_bf16_decode_closed_forms_and_permutation():
    case = W.make_paged_case(batch=3, num_q_heads=4, num_kv_heads=1, head_dim=16,
                             context_lens=[1, 20, 0], seed=15, permute=False)
    kc, vc = W.paged_bf16_cache(case)
    out = O.paged_decode_bf16(case.q, kc, vc, case.block_table, case.context_lens)
    v0 = case.v[case.token_seq == 0][0, 0].astype(np.float64)
    for h in range(4):
        assert np.array_equal(out[0, h], v0)           # single token: its V
    assert np.all(out[2] == 0)                         # empty context
    blk = case.block_table[1]
    for t in range(20):                                # identical keys: mean V
        kc[blk[t // 16], 0, t % 16] = kc[blk[0], 0, 0]
    out = O.paged_decode_bf16(case.q, kc, vc, case.block_table, case.context_lens)
    vmean = case.v[case.token_seq == 1][:, 0].astype(np.float64).mean(axis=0)
    assert np.allclose(out[1], vmean[None, :], rtol=1e-13, atol=1e-14)
    perm = np.random.default_rng(2).permutation(case.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    out2 = O.paged_decode_bf16(case.q, kc2, vc2, perm[case.block_table], case.context_lens)
    assert np.array_equal(out2, out)


def test_bf16_decode_equals_int8_decode_on_exact_values():
    """With every scale 2^-6, code * scale is exact in bf16, so a bf16 cache
    holding those values must give the INT8 path's result: the two gathers
    and the shared attention definition agree."""
    case = W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=16,
                             context_lens=[7, 40, 129], q_dtype="f32", seed=16)
    kc, vc, ks, vs = build_cache(case)
    ks[:] = np.float16(2.0 ** -6)
    vs[:] = np.float16(2.0 ** -6)
    ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    _, kb = W.to_bf16(kc.astype(np.float32) * np.float32(2.0 ** -6))
    _, vb = W.to_bf16(vc.astype(np.float32) * np.float32(2.0 ** -6))
    assert np.array_equal(W.bf16_bits_to_f32(kb), kc.astype(np.float32) / 64)   # exact
    out = O.paged_decode_bf16(case.q, kb, vb, case.block_table, case.context_lens)
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# FP8 (e4m3) cache ("KV Cache 优化全景解析" section 7.4).  torch's
# float8_e4m3fn is an independent implementation of the OCP e4m3 format: it
# decodes every code and rounds to nearest even below the saturation point
# (464 and above it gives NaN, where the quantiser saturates to 448).
# ---------------------------------------------------------------------------
def torch_e4m3(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_fp8_decode_every_code_vs_torch():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_value(c)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_fp8_encode_every_bf16_vs_torch_and_saturation():
    x = W.bf16_bits_to_f32(np.arange(0x10000, dtype=np.uint32).astype(np.uint16))
    x = x[np.isfinite(x)]
    got = O.e4m3_encode(x)
    inr = np.abs(x) < 464
    assert np.array_equal(got[inr], torch_e4m3(x[inr]))
    sat = ~inr
    assert np.all(got[sat] == np.where(x[sat] < 0, 0xFE, 0x7E))
    assert not np.any((got & 0x7F) == 0x7F)           # never NaN


def test_fp8_encode_random_fp32_and_ties_vs_torch():
    rng = np.random.default_rng(21)
    x = np.concatenate([
        rng.uniform(-463.9, 463.9, 200000), rng.uniform(-1, 1, 200000) * 2.0 ** -5,
        rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 9, 200000),
    ]).astype(np.float32)
    # exact midpoints between neighbouring codes (ties go to the even code)
    vals = O.e4m3_value(np.arange(0, 0x7E, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    got = O.e4m3_encode(x)
    inr = np.abs(x) < 464
    assert np.array_equal(got[inr], torch_e4m3(x[inr]))
    assert np.all(got[~inr] == np.where(x[~inr] < 0, 0xFE, 0x7E))


def test_fp8_quantiser_invariants():
    rng = np.random.default_rng(22)
    rows = rng.standard_normal((2000, 64)).astype(np.float32) * \
        np.exp2(rng.integers(-20, 12, 2000)).astype(np.float32)[:, None]
    _, rows = W.to_bf16(rows)
    rows = W.bf16_bits_to_f32(rows)
    codes, s = O.quantize_rows_fp8(rows)
    s64 = s.astype(np.float64)
    i = np.argmax(np.abs(rows), axis=1)
    top = codes[np.arange(len(rows)), i]
    normal = s64 >= 2.0 ** -14                        # scale not subnormal
    assert np.all((top[normal] & 0x7F) == 0x7E)       # the absmax lands on +-448
    xhat = O.dequantize_rows_fp8(codes, s)
    err = np.abs(xhat - rows)
    # half an e4m3 step: 2^-4 relative above 2^-6 * s, 2^-10 * s below
    bound = np.maximum(np.abs(rows) * 2.0 ** -4, 2.0 ** -10 * s64[:, None])
    assert np.all(err[normal] <= bound[normal] * (1 + 1e-12))
    z, sz = O.quantize_rows_fp8(np.zeros((3, 16), np.float32))
    assert np.all(z == 0) and np.all(sz == 0)
    neg, _ = O.quantize_rows_fp8(-rows)
    nz = s64 > 0                                      # zero-scale rows are all 0x00
    assert np.array_equal((neg ^ 0x80)[nz], codes[nz])   # symmetric, signed zero kept
    assert np.all(codes[~nz] == 0) and np.all(neg[~nz] == 0)


def test_fp8_scale_every_bf16_absmax():
    """Every positive finite bf16 absmax against exact rational rounding of
    absmax / 448 to fp16 (nearest even, gradual underflow), saturated to
    65504: covers the underflow band (scale 0), the subnormal scales and the
    saturation band (absmax >= 448 * 65520)."""
    a = all_finite_bf16(positive_only=True)
    got = O.row_scale_fp8(a[:, None]).astype(np.float64)
    exp = []
    for v in a.tolist():
        s = fp16_rne_exact(Fraction(v) / 448)
        exp.append(65504.0 if s == math.inf else s)
    exp = np.array(exp)
    assert np.array_equal(got, exp)
    assert np.count_nonzero(exp == 0) > 0                       # underflow band present
    assert np.count_nonzero((exp > 0) & (exp < 2.0 ** -14)) > 0   # subnormal scales
    assert np.count_nonzero(a >= 448.0 * 65520) > 1000           # saturation band


def e4m3_grid():
    """The 127 non-negative finite e4m3 values in code order, from the
    format's definition (bias 7, 3 mantissa bits, subnormals m * 2^-9, code
    0x7F reserved): fp64, exact."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    return np.array(vals)


def exact_e4m3_codes(x, s):
    """e4m3 codes of x / s by exact comparison against the exact midpoints
    s * (v_k + v_{k+1}) / 2 (each a product of a 5-bit and an 11-bit
    significand, so exact in fp64); ties go to the even code; beyond the
    last midpoint everything is 448 (code 0x7E); the sign of x is kept."""
    x = np.asarray(x, np.float64)
    if s == 0:
        return np.zeros(x.shape, np.int64)
    grid = e4m3_grid()
    thr = float(s) * (grid[:-1] + grid[1:]) / 2
    a = np.abs(x)
    k = np.searchsorted(thr, a, side="left")           # number of midpoints below a
    tie = (k < len(thr)) & (thr[np.minimum(k, len(thr) - 1)] == a)
    k = np.where(tie & (k % 2 == 1), k + 1, k)          # tie between k and k+1: even code
    return np.where(np.signbit(x), 0x80, 0) | k


FP8_SCALES = [1.0, 3.0, 3.5, 0.0234375, 2.0 ** -14, 3 * 2 ** -24, 1000 * 2 ** -24, 65504.0,
              1.5 * 2.0 ** 10]


@pytest.mark.parametrize("s", FP8_SCALES)
def test_fp8_codes_every_bf16(s):
    """Every finite bf16 x (both signs, zeros, subnormals, values whose
    quotient saturates) under normal, subnormal and saturated scales against
    exact rounding onto the e4m3 grid.  At s = 3 the bf16 grid holds exact
    midpoints x / s (5-bit midpoints times 3), so tie handling is decided
    exactly; at s = 3.5 a quotient taken as x * fp32(1/s) rounds 60 values
    differently; a quotient rounded through fp16 fails at large |x|."""
    x = all_finite_bf16()
    got = O.codes_fp8_for_scale(x[None, :], np.array([s], np.float16))[0].astype(np.int64)
    exp = exact_e4m3_codes(x, float(np.float16(s)))
    assert np.array_equal(got, exp)
    if s == 3.0:
        grid = e4m3_grid()
        mids = 3.0 * (grid[:-1] + grid[1:]) / 2
        assert np.count_nonzero(np.isin(np.abs(x), mids)) > 50   # ties really occur


def test_fp8_exact_reference_vs_fraction():
    """The exact e4m3 reference above against Fraction arithmetic on a
    random sample plus every exact midpoint at s = 3."""
    grid = [Fraction(v) for v in e4m3_grid().tolist()]

    def frac_code(xv, s):
        q = abs(Fraction(xv) / Fraction(s))
        best = None
        for k, v in enumerate(grid):
            d = abs(q - v)
            if best is None or d < best[0] or (d == best[0] and k % 2 == 0):
                best = (d, k)
        return (0x80 if math.copysign(1.0, xv) < 0 else 0) | best[1]

    x = all_finite_bf16()
    rng = np.random.default_rng(25)
    for s in (3.0, 1000 * 2 ** -24, 65504.0):
        pick = x[rng.choice(len(x), 400, replace=False)]
        if s == 3.0:
            g = e4m3_grid()
            mids = 3.0 * (g[:-1] + g[1:]) / 2
            pick = np.concatenate([pick, x[np.isin(np.abs(x), mids)]])
        exp = exact_e4m3_codes(pick, s)
        for xv, e in zip(pick.tolist(), exp.tolist()):
            assert frac_code(xv, s) == e


def build_cache_fp8(case):
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, case.num_kv_heads, case.head_dim)
    kc, vc = kc.view(np.uint8), vc.view(np.uint8)
    O.quant_append_fp8(case.k, case.v, case.slot_mapping, kc, vc, ks, vs)
    return kc, vc, ks, vs


def test_fp8_decode_brute_force_and_sdpa():
    case = W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=16,
                             context_lens=[1, 37, 130], q_dtype="f32", k_outliers=True, seed=23)
    kc, vc, ks, vs = build_cache_fp8(case)
    out = O.paged_decode_fp8(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    for b in range(3):
        rk = case.k[case.token_seq == b]
        rv = case.v[case.token_seq == b]
        K = O.dequantize_rows_fp8(*O.quantize_rows_fp8(rk))
        V = O.dequantize_rows_fp8(*O.quantize_rows_fp8(rv))
        for h in range(8):
            ref = brute_attention(case.q[b, h], K[:, h // 4], V[:, h // 4], 1 / math.sqrt(16))
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)
    v0 = O.gather_dequant_fp8(vc, vs, case.block_table[0], 1, 0)[0]
    assert np.array_equal(out[0, 0], v0)              # single token: its V


def test_fp8_prefill_equals_sdpa_causal():
    case = W.prefill_case([0, 9], [21, 40], num_q_heads=4, num_kv_heads=2, head_dim=16, seed=24)
    kc, vc, ks, vs = build_cache_fp8(case)
    out = O.paged_prefill_chunk_fp8(case.q, case.extra["q_start_loc"], kc, vc, ks, vs,
                                    case.block_table, case.context_lens)
    qsl = case.extra["q_start_loc"]
    for b in range(2):
        ctx = int(case.context_lens[b])
        K = np.stack([O.gather_dequant_fp8(kc, ks, case.block_table[b], ctx, g) for g in range(2)])
        V = np.stack([O.gather_dequant_fp8(vc, vs, case.block_table[b], ctx, g) for g in range(2)])
        lc = qsl[b + 1] - qsl[b]
        q = torch.from_numpy(case.q[qsl[b]:qsl[b + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        Kt = torch.from_numpy(K).repeat_interleave(2, dim=0)[None]
        Vt = torch.from_numpy(V).repeat_interleave(2, dim=0)[None]
        pos = ctx - lc + np.arange(lc)
        mask = torch.from_numpy(np.arange(ctx)[None, :] <= pos[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, attn_mask=mask)
        assert np.allclose(out[qsl[b]:qsl[b + 1]], ref[0].permute(1, 0, 2).numpy(),
                           rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# RoPE fused into the append (README section 系统架构概览; rotate-half
# reading).  transformers' apply_rotary_pos_emb is an independent
# implementation of the same convention.
# ---------------------------------------------------------------------------
def rope_table(max_pos, d, base=500000.0):
    inv = 1.0 / base ** (np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def test_rope_matches_transformers_and_fp64():
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    rng = np.random.default_rng(41)
    n, h, d = 300, 4, 128
    tab = rope_table(70000, d)
    pos = rng.integers(0, 70000, n)
    x = W.bf16_bits_to_f32(W.to_bf16(rng.standard_normal((n, h, d)).astype(np.float32) * 3)[1])
    got = O.rope_rotate_half(x, pos, tab)
    c = torch.from_numpy(np.concatenate([tab[pos, :d // 2]] * 2, axis=1))      # [n, d]
    s = torch.from_numpy(np.concatenate([tab[pos, d // 2:]] * 2, axis=1))
    xt = torch.from_numpy(x)
    ref, _ = apply_rotary_pos_emb(xt, xt, c, s, unsqueeze_dim=1)
    ulp = np.spacing(np.abs(ref.numpy()).astype(np.float32))
    assert np.all(np.abs(got - ref.numpy()) <= ulp)        # same rounded ops, at most 1 ulp
    # against the exact rotation with the same table (fp64): within 2 fp32 ulps
    t64 = tab[pos].astype(np.float64)
    c64, s64 = t64[:, None, :d // 2], t64[:, None, d // 2:]
    lo, hi = x[..., :d // 2].astype(np.float64), x[..., d // 2:].astype(np.float64)
    exact = np.concatenate([lo * c64 - hi * s64, hi * c64 + lo * s64], axis=-1)
    # each fp32 product rounds by half an ulp of itself, the sum by half an ulp of the result
    sp = lambda v: np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)
    pa = np.concatenate([lo * c64, hi * c64], axis=-1)
    pb = np.concatenate([hi * s64, lo * s64], axis=-1)
    bound = 0.5 * (sp(pa) + sp(pb) + sp(exact)) * (1 + 1e-9)
    assert np.all(np.abs(got - exact) <= bound)


def test_rope_identity_at_zero_and_relative_position():
    rng = np.random.default_rng(42)
    d = 64
    tab = rope_table(5000, d, base=10000.0)
    x = rng.standard_normal((1, 1, d)).astype(np.float32)
    assert np.array_equal(O.rope_rotate_half(x, [0], tab), x)        # cos 1, sin 0
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, d)).astype(np.float32)
    dots = []
    for m, n_ in ((100, 40), (1060, 1000), (60, 0)):
        dots.append(float(np.dot(O.rope_rotate_half(q, [m], tab).ravel().astype(np.float64),
                                 O.rope_rotate_half(k, [n_], tab).ravel().astype(np.float64))))
    assert np.allclose(dots, dots[0], rtol=1e-4, atol=1e-4)          # depends on m - n only
    norms = np.linalg.norm(O.rope_rotate_half(x, [1234], tab)), np.linalg.norm(x)
    assert abs(norms[0] - norms[1]) < 1e-5 * norms[1]                 # a rotation


def test_rope_quant_append_is_rotate_then_quantise():
    case = W.make_paged_case(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
                             context_lens=[20, 33], seed=43)
    tab = rope_table(4096, 64)
    pos = case.token_pos + 7
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, 2, 64)
    O.rope_quant_append(case.k, case.v, pos, tab, case.slot_mapping, kc, vc, ks, vs)
    kq, ksc = O.quantize_rows(O.rope_rotate_half(case.k, pos, tab))
    vq, vsc = O.quantize_rows(case.v)
    blk, off = case.slot_mapping // 16, case.slot_mapping % 16
    assert np.array_equal(kc[blk, :, off], kq) and np.array_equal(vc[blk, :, off], vq)
    assert np.array_equal(ks[blk, :, off], ksc) and np.array_equal(vs[blk, :, off], vsc)


# ---------------------------------------------------------------------------
# INT4 cache (KV-size table of "KV Cache 优化全景解析" section 2.3: INT4 = 0.5 B;
# reading: the INT8 recipe with 7 in place of 127, two's-complement nibbles)
# ---------------------------------------------------------------------------
def exact_codes_q(x, s, qmax):
    """round_half_even(x / s) clamped to +-qmax by exact rational arithmetic."""
    if s == 0:
        return np.zeros(len(x), np.int64)
    out = []
    for xv in np.asarray(x, np.float64).tolist():
        q = round(Fraction(xv) / Fraction(float(s)))
        out.append(max(-qmax, min(qmax, q)))
    return np.array(out, np.int64)


def test_int4_scale_every_bf16_absmax():
    a = all_finite_bf16(positive_only=True)
    got = O.row_scale_int4(a[:, None]).astype(np.float64)
    exp = []
    for v in a.tolist():
        e = fp16_rne_exact(Fraction(v) / 7)
        exp.append(65504.0 if e == math.inf else e)
    assert np.array_equal(got, np.array(exp))


@pytest.mark.parametrize("s", [1.0, 0.0234375, 3 * 2 ** -24, 2.0 ** -14, 9362.0])
def test_int4_codes_every_bf16(s):
    x = all_finite_bf16()
    got = O.codes_int4_for_scale(x[None, :], np.array([s], np.float16))[0].astype(np.int64)
    # exact rational rounding, on every value whose quotient is within the
    # clamp (+-7.5) and on a sample beyond it
    q = np.abs(x.astype(np.float64)) / s
    near = np.nonzero(q < 16)[0]
    far = np.nonzero(q >= 16)[0]
    far = far[np.random.default_rng(52).choice(len(far), min(300, len(far)), replace=False)]
    for idx in (near, far):
        assert np.array_equal(got[idx], exact_codes_q(x[idx], np.float16(s), 7))


def test_int4_packing_worked_example_and_roundtrip():
    codes = np.array([[-7, 7, 0, -1, 1, -2, 5, 3]], np.int8)
    packed = O.pack_int4(codes)
    # byte i = (code 2i+1 & 0xF) << 4 | (code 2i & 0xF)
    assert packed.tolist() == [[0x79, 0xF0, 0xE1, 0x35]]
    assert np.array_equal(O.unpack_int4(packed), codes)
    rng = np.random.default_rng(53)
    c = rng.integers(-7, 8, size=(100, 64)).astype(np.int8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(c)), c)


def test_int4_quantiser_invariants():
    rng = np.random.default_rng(54)
    rows, _ = W.to_bf16(rng.standard_normal((500, 128)).astype(np.float32))
    p, s = O.quantize_rows_int4(rows)
    c = O.unpack_int4(p)
    am = np.argmax(np.abs(rows), axis=1)
    assert np.all(np.abs(c[np.arange(500), am]) == 7) and c.min() >= -7 and c.max() <= 7
    err = np.abs(rows - O.dequantize_rows_int4(p, s))
    assert np.all(err <= s.astype(np.float64)[:, None] / 2)
    pn, sn = O.quantize_rows_int4(-rows)
    assert np.array_equal(O.unpack_int4(pn), -c) and np.array_equal(sn, s)


def build_cache_int4(case):
    kc, vc, ks, vs = O.alloc_paged_cache_int4(case.num_blocks, case.num_kv_heads, case.head_dim)
    O.quant_append_int4(case.k, case.v, case.slot_mapping, kc, vc, ks, vs)
    return kc, vc, ks, vs


def test_int4_decode_and_prefill_brute_force():
    case = W.make_paged_case(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=16,
                             context_lens=[5, 37], q_dtype="f32", seed=55)
    kc, vc, ks, vs = build_cache_int4(case)
    out = O.paged_decode_int4(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    for b in range(2):
        K = O.dequantize_rows_int4(*O.quantize_rows_int4(case.k[case.token_seq == b]))
        V = O.dequantize_rows_int4(*O.quantize_rows_int4(case.v[case.token_seq == b]))
        for h in range(4):
            ref = brute_attention(case.q[b, h], K[:, h // 2], V[:, h // 2], 1 / math.sqrt(16))
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)
    pc = W.prefill_case([0, 9], [21, 40], num_q_heads=4, num_kv_heads=2, head_dim=16, seed=56)
    kc, vc, ks, vs = build_cache_int4(pc)
    pout = O.paged_prefill_chunk_int4(pc.q, pc.extra["q_start_loc"], kc, vc, ks, vs,
                                      pc.block_table, pc.context_lens)
    qsl = pc.extra["q_start_loc"]
    for b in range(2):
        ctx = int(pc.context_lens[b])
        K = O.gather_dequant_int4(kc, ks, pc.block_table[b], ctx, 1)
        V = O.gather_dequant_int4(vc, vs, pc.block_table[b], ctx, 1)
        lc = qsl[b + 1] - qsl[b]
        for i in (0, lc - 1):
            pos = ctx - lc + i
            ref = brute_attention(pc.q[qsl[b] + i, 3], K[:pos + 1], V[:pos + 1], 1 / math.sqrt(16))
            assert np.allclose(pout[qsl[b] + i, 3], ref, rtol=1e-12, atol=1e-13)
