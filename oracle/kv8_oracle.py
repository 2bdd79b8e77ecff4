"""Plain fp64 CPU oracle for paged INT8-KV GQA attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check of the package entry
and the CPU-baseline leg of the benchmark use it.  It shares no code, table or
helper with the HIP library; both sides receive their inputs from the seeded
generators, which hold none of the method's arithmetic.

What it computes, and where each step comes from
------------------------------------------------
Sources are the pages collected for this method:

* [P1] "KV-Cache 全栈优化系统" (project README on gitlink), section
  "主要特性" (main features), item on low-bit linear and KV-cache
  compression: the attention layer keeps K/V as INT8 obtained by dynamic
  per-token quantisation and restores them on demand during attention.
* [P3] "KV Cache 优化全景解析——从基础原理到工程实践" (cnblogs daily report):
  section 2.1, the attention equation softmax(Q K^T / sqrt(d_k)) V;
  section 2.3, the KV-cache size formula 2 x L x B x T x H_kv x d_h x bytes
  with INT8 = 1 byte; section 3.3, GQA: the query heads are split into groups
  and every group shares one K/V head; section 4.2, PagedAttention: logical
  blocks are mapped to physical blocks through a block table; section 6.3,
  vLLM hashes fixed blocks of 16/32 tokens.
* [P4] "大模型推理加速：KV Cache与vLLM技术解析" section 4.1: KV cache kept in
  FP16/INT8 while attention accumulates in FP32.

The pages do not spell out the quantiser's arithmetic.  The readings taken
here:

1. one scale per (token, KV head), separately for K and V;
2. scale s = fp16_rne(fp32_rne(absmax / 127)), gradual underflow, an fp16
   overflow saturates to 65504;
3. codes c_i = clamp(round_half_even(fp32_rne(x_i / s)), -127, 127), all
   zero when s == 0;
4. dequantised value x_hat_i = c_i * s (exact in fp64);
5. attention runs in fp64 over the dequantised cache; head h of Hq reads KV
   head h // (Hq / Hkv); logical token t of a sequence lives in physical block
   block_table[b, t // 16] at slot t % 16; an empty context yields zeros;
6. a prefill chunk of Lc rows for a sequence with ctx tokens (chunk
   included) places row i at absolute position ctx - Lc + i, which attends to
   keys 0 .. ctx - Lc + i inclusive.

The code step divides in fp32 exactly as specified, so the integer decision
is taken in the same precision as the GPU.  For bf16 inputs and fp16 scales
the fp32 rounding of the quotient can never move a non-tie onto a tie (the
quotient of an 8-bit-significand value by an 11-bit-significand value is at
least 2^-12 away from any half-integer it does not equal, far above fp32's
half-ulp below 128), so the result equals exact rational rounding; the pin
tests check that exhaustively.

Every function here is written for clarity, not speed.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16          # tokens per physical block ([P3] section 6.3)
QMAX = 127               # symmetric INT8 range, -128 never produced
FP16_MAX = 65504.0       # largest finite fp16, used when the scale overflows


# --------------------------------------------------------------------------
# KV-cache size ([P3] section 2.3 formula and its symbol table)
# --------------------------------------------------------------------------
def kv_cache_bytes(num_layers, batch, seq_len, num_kv_heads, head_dim,
                   bytes_per_elem):
    """Closed form 2 * L * B * T * H_kv * d_h * bytes ([P3] section 2.3)."""
    return 2 * num_layers * batch * seq_len * num_kv_heads * head_dim * bytes_per_elem


def paged_cache_bytes(num_blocks, num_kv_heads, head_dim, block_size=BLOCK_SIZE):
    """Bytes held by one layer of the paged INT8 cache: K and V codes
    (1 byte each) plus one fp16 scale per (token slot, KV head) for K and V."""
    slots = num_blocks * block_size * num_kv_heads
    return 2 * slots * head_dim * 1 + 2 * slots * 2


def alloc_paged_cache(num_blocks, num_kv_heads, head_dim, block_size=BLOCK_SIZE):
    """Zeroed cache arrays in the layout the library uses:
    codes [NB, Hkv, block_size, d] int8 and scales [NB, Hkv, block_size]
    fp16, for K and for V."""
    kc = np.zeros((num_blocks, num_kv_heads, block_size, head_dim), np.int8)
    vc = np.zeros_like(kc)
    ks = np.zeros((num_blocks, num_kv_heads, block_size), np.float16)
    vs = np.zeros_like(ks)
    return kc, vc, ks, vs


# --------------------------------------------------------------------------
# Per-token INT8 quantiser ([P1] main features; readings 1-4 above)
# --------------------------------------------------------------------------
def row_scale(x):
    """fp16 scale of each row of x (last axis = channels of one token and
    head): absmax / 127, rounded to fp32 then to fp16 (round to nearest
    even, gradual underflow), saturated to 65504 on overflow."""
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)   # exact: inputs are bf16
    s32 = a / np.float32(QMAX)                            # IEEE fp32 divide, RNE
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)                      # RNE, subnormals kept
    return np.where(np.isinf(s16), np.float16(FP16_MAX), s16).astype(np.float16)


def codes_for_scale(x, s):
    """INT8 codes of x (rows along the last axis) under fp16 scales s (one
    per row): fp32 quotient, round half to even, clamp to [-127, 127];
    rows whose scale is zero give all-zero codes."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = x32 / np.where(zero, np.float32(1), s32)   # IEEE fp32 divide
    q = np.rint(quot.astype(np.float64))                  # half to even
    q = np.clip(q, -QMAX, QMAX)
    q = np.where(zero, 0.0, q)
    return q.astype(np.int8)


def quantize_rows(x):
    """Quantise each row of x (shape [..., d]) to (codes int8 [..., d],
    scales fp16 [...])."""
    s = row_scale(x)
    return codes_for_scale(x, s), s


def dequantize_rows(codes, scales):
    """x_hat = code * scale, exact in fp64."""
    return codes.astype(np.float64) * np.asarray(scales, np.float16).astype(np.float64)[..., None]


# --------------------------------------------------------------------------
# Append: quantise new tokens and scatter them into the paged cache
# ([P1] main features: quantised as they are written; [P3] section 4.2)
# --------------------------------------------------------------------------
def slot_to_block(slot, block_size=BLOCK_SIZE):
    """Physical slot -> (physical block, offset inside the block)."""
    return slot // block_size, slot % block_size


def quant_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                 block_size=BLOCK_SIZE):
    """k_new, v_new: [N, Hkv, d] bf16 values (as float arrays); slot_mapping
    [N] int, negative entries are skipped.  Writes codes and scales in place
    and returns nothing.  Repeated slots are the caller's error."""
    kc, ks = quantize_rows(k_new)
    vc, vs = quantize_rows(v_new)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = slot_to_block(slot, block_size)
        k_cache[blk, :, off, :] = kc[n]
        v_cache[blk, :, off, :] = vc[n]
        k_scale[blk, :, off] = ks[n]
        v_scale[blk, :, off] = vs[n]


# --------------------------------------------------------------------------
# Paged attention ([P3] sections 2.1, 3.3, 4.2)
# --------------------------------------------------------------------------
def kv_head_of(h, group):
    """Query head h reads KV head h // G (contiguous grouping)."""
    return h // group


def logical_to_physical(block_table_row, t, block_size=BLOCK_SIZE):
    """Logical token t -> (physical block id, slot in block)."""
    return block_table_row[t // block_size], t % block_size


def gather_dequant(codes, scales, block_table_row, ctx, kv_head,
                   block_size=BLOCK_SIZE):
    """Dequantised [ctx, d] fp64 matrix of one sequence and one KV head,
    read through the block table."""
    t = np.arange(ctx)
    blk, off = logical_to_physical(np.asarray(block_table_row), t, block_size)
    return dequantize_rows(codes[blk, kv_head, off, :], scales[blk, kv_head, off])


def softmax_attention(q_rows, k, v, sm_scale, visible=None):
    """softmax(q k^T * sm_scale) v in fp64 with the max subtracted first.
    visible: optional boolean [rows, T] mask of the keys each row may see."""
    scores = (q_rows @ k.T) * sm_scale
    if visible is not None:
        scores = np.where(visible, scores, -np.inf)
    m = np.max(scores, axis=-1, keepdims=True)
    p = np.exp(scores - m)
    return (p @ v) / np.sum(p, axis=-1, keepdims=True)


def paged_decode(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                 sm_scale=None, block_size=BLOCK_SIZE):
    """One query token per sequence.  q [B, Hq, d]; returns fp64 [B, Hq, d]."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        for h in range(Hq):
            g = kv_head_of(h, G)
            k = gather_dequant(k_cache, k_scale, block_table[b], ctx, g, block_size)
            v = gather_dequant(v_cache, v_scale, block_table[b], ctx, g, block_size)
            out[b, h] = softmax_attention(q[b, h][None, :], k, v, sm_scale)[0]
    return out


def causal_visibility(ctx, lc):
    """[lc, ctx] mask: row i (absolute position ctx - lc + i) sees keys at
    positions 0 .. ctx - lc + i inclusive."""
    pos = ctx - lc + np.arange(lc)
    return np.arange(ctx)[None, :] <= pos[:, None]


def paged_prefill_chunk(q, q_start_loc, k_cache, v_cache, k_scale, v_scale,
                        block_table, context_lens, sm_scale=None,
                        block_size=BLOCK_SIZE):
    """Causal chunk attention over a paged cache that already holds the
    chunk's own K/V.  q [Tq, Hq, d] with sequence b's rows at
    q_start_loc[b] .. q_start_loc[b+1]-1; context_lens[b] counts every token
    of sequence b, chunk included.  Returns fp64 [Tq, Hq, d]."""
    q = np.asarray(q, np.float64)
    Tq, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((Tq, Hq, d), np.float64)
    B = len(context_lens)
    for b in range(B):
        r0, r1 = int(q_start_loc[b]), int(q_start_loc[b + 1])
        lc = r1 - r0
        ctx = int(context_lens[b])
        if lc <= 0 or ctx <= 0:
            continue
        visible = causal_visibility(ctx, lc)
        for h in range(Hq):
            g = kv_head_of(h, G)
            k = gather_dequant(k_cache, k_scale, block_table[b], ctx, g, block_size)
            v = gather_dequant(v_cache, v_scale, block_table[b], ctx, g, block_size)
            out[r0:r1, h] = softmax_attention(q[r0:r1, h], k, v, sm_scale, visible)
    return out


# --------------------------------------------------------------------------
# 16-bit KV reference point.  [P1] section "实验效果（摘要）" compares KV8
# attention with FlashAttention-2 over the unquantised cache when both get
# the same GPU-memory budget; the 16-bit side is plain attention over the
# paged bf16 cache ([P3] sections 2.1, 3.3, 4.2), no quantiser involved.
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values (a bf16 value is the
    fp32 whose upper 16 bits are the pattern)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def gather_bf16(cache_bits, block_table_row, ctx, kv_head, block_size=BLOCK_SIZE):
    """[ctx, d] fp64 rows of one sequence and one KV head of a paged bf16
    cache [NB, Hkv, block_size, d] (bit patterns), read through the block
    table."""
    t = np.arange(ctx)
    blk, off = logical_to_physical(np.asarray(block_table_row), t, block_size)
    return bf16_bits_to_f64(cache_bits[blk, kv_head, off, :])


def paged_decode_bf16(q, k_cache_bits, v_cache_bits, block_table, context_lens,
                      sm_scale=None, block_size=BLOCK_SIZE):
    """One query token per sequence over a paged bf16 cache.  q [B, Hq, d];
    returns fp64 [B, Hq, d]; an empty context yields zeros."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache_bits.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        for h in range(Hq):
            g = kv_head_of(h, G)
            k = gather_bf16(k_cache_bits, block_table[b], ctx, g, block_size)
            v = gather_bf16(v_cache_bits, block_table[b], ctx, g, block_size)
            out[b, h] = softmax_attention(q[b, h][None, :], k, v, sm_scale)[0]
    return out


# --------------------------------------------------------------------------
# FP8 (e4m3) KV cache.  "KV Cache 优化全景解析" section 7.4: the KV cache kept
# as FP8, e4m3 (4 exponent bits, 3 mantissa bits, the more precise of the two
# formats) with quantisation scales; section 11.3: about half the bytes of a
# 16-bit cache.  Readings taken: the OCP e4m3 format
# (bias 7, subnormals, largest finite 448, no infinity); one fp16 scale per
# (token, KV head) as for INT8, s = fp16_rne(fp32_rne(absmax / 448));
# codes = e4m3 round-to-nearest-even of the fp32 quotient x / s, saturated
# to +-448; all-zero codes when s == 0; x_hat = e4m3 value * s.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_value(codes):
    """fp64 value of e4m3 codes (uint8): sign bit 7, exponent bits 6..3
    (bias 7), mantissa bits 2..0; exponent 0 holds the subnormals
    m * 2^-9; the two all-ones patterns 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """e4m3 codes of fp32 values x: round to nearest, ties to even, on the
    exact grid (spacing 2^(e-3) for |x| in [2^e, 2^(e+1)), e >= -6; spacing
    2^-9 below 2^-6), then saturate to +-448.  Zero keeps its sign."""
    x = np.asarray(x, np.float32).astype(np.float64)
    # saturation first: every magnitude at or above 448 (an overflowed,
    # infinite quotient included) codes as 448, and below it rounding to the
    # grid never exceeds 448, so clamping before rounding is the same rule
    a = np.minimum(np.abs(x), E4M3_MAX)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    ulp = np.exp2(e - 3)
    r = np.rint(a / ulp) * ulp                 # exact: power-of-two scaling, RNE
    # code of the rounded magnitude r (a grid point or 448)
    sub = r < 2.0 ** -6
    ee = np.where(sub, 0, np.floor(np.log2(np.where(sub, 1.0, r))) + 7).astype(np.int64)
    mm = np.where(sub, np.rint(r / 2.0 ** -9),
                  np.rint(r / np.exp2(ee.astype(np.float64) - 7) * 8) - 8).astype(np.int64)
    code = (ee << 3) | mm
    return (np.where(np.signbit(x), 0x80, 0) | code).astype(np.uint8)


def row_scale_fp8(x):
    """fp16 scale of each row for FP8 codes: absmax / 448 rounded to fp32
    then fp16 (nearest even, gradual underflow), saturated to 65504."""
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    s32 = a / np.float32(E4M3_MAX)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    return np.where(np.isinf(s16), np.float16(FP16_MAX), s16).astype(np.float16)


def codes_fp8_for_scale(x, s):
    """e4m3 codes of rows x under fp16 scales s: IEEE fp32 quotient, then
    e4m3_encode; rows with a zero scale give all-zero codes."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = x32 / np.where(zero, np.float32(1), s32)
    codes = e4m3_encode(quot)
    return np.where(zero, np.uint8(0), codes).astype(np.uint8)


def quantize_rows_fp8(x):
    s = row_scale_fp8(x)
    return codes_fp8_for_scale(x, s), s


def dequantize_rows_fp8(codes, scales):
    """x_hat = e4m3 value * scale, exact in fp64."""
    return e4m3_value(codes) * np.asarray(scales, np.float16).astype(np.float64)[..., None]


def quant_append_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                     block_size=BLOCK_SIZE):
    """As quant_append, with e4m3 codes (uint8 caches)."""
    kc, ks = quantize_rows_fp8(k_new)
    vc, vs = quantize_rows_fp8(v_new)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = slot_to_block(slot, block_size)
        k_cache[blk, :, off, :] = kc[n]
        v_cache[blk, :, off, :] = vc[n]
        k_scale[blk, :, off] = ks[n]
        v_scale[blk, :, off] = vs[n]


def gather_dequant_fp8(codes, scales, block_table_row, ctx, kv_head, block_size=BLOCK_SIZE):
    t = np.arange(ctx)
    blk, off = logical_to_physical(np.asarray(block_table_row), t, block_size)
    return dequantize_rows_fp8(codes[blk, kv_head, off, :], scales[blk, kv_head, off])


def paged_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                     sm_scale=None, block_size=BLOCK_SIZE):
    """paged_decode over an e4m3 cache.  Returns fp64 [B, Hq, d]."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    G = Hq // k_cache.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        for h in range(Hq):
            g = kv_head_of(h, G)
            k = gather_dequant_fp8(k_cache, k_scale, block_table[b], ctx, g, block_size)
            v = gather_dequant_fp8(v_cache, v_scale, block_table[b], ctx, g, block_size)
            out[b, h] = softmax_attention(q[b, h][None, :], k, v, sm_scale)[0]
    return out


def paged_prefill_chunk_fp8(q, q_start_loc, k_cache, v_cache, k_scale, v_scale,
                            block_table, context_lens, sm_scale=None, block_size=BLOCK_SIZE):
    """paged_prefill_chunk over an e4m3 cache.  Returns fp64 [Tq, Hq, d]."""
    q = np.asarray(q, np.float64)
    Tq, Hq, d = q.shape
    G = Hq // k_cache.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((Tq, Hq, d), np.float64)
    for b in range(len(context_lens)):
        r0, r1 = int(q_start_loc[b]), int(q_start_loc[b + 1])
        lc, ctx = r1 - r0, int(context_lens[b])
        if lc <= 0 or ctx <= 0:
            continue
        visible = causal_visibility(ctx, lc)
        for h in range(Hq):
            g = kv_head_of(h, G)
            k = gather_dequant_fp8(k_cache, k_scale, block_table[b], ctx, g, block_size)
            v = gather_dequant_fp8(v_cache, v_scale, block_table[b], ctx, g, block_size)
            out[r0:r1, h] = softmax_attention(q[r0:r1, h], k, v, sm_scale, visible)
    return out


# --------------------------------------------------------------------------
# RoPE fused into the append.  "KV-Cache 全栈优化系统" README, section
# 系统架构概览: on the cache-operator plane K is written to the cache after
# RoPE, then quantised.  The pages give no RoPE formula; the reading taken is
# the standard rotary embedding in the rotate-half (Llama) convention over
# the whole head: for j < d/2, with (c, s) = table[pos, j], table[pos, d/2+j],
#   x'_j       = x_j * c - x_{j+d/2} * s
#   x'_{j+d/2} = x_{j+d/2} * c + x_j * s
# in fp32, each product and the sum rounded to fp32 (no fused multiply-add),
# so the quantiser sees fp32 values.  The cos/sin table [max_pos, d] is an
# input, as in serving engines.  V is not rotated.
# --------------------------------------------------------------------------
def rope_rotate_half(x, positions, cos_sin):
    """x [N, H, d] (fp32 values), positions [N] int, cos_sin [P, d] fp32.
    Returns the rotated rows as fp32."""
    x = np.asarray(x, np.float32)
    d = x.shape[-1]
    half = d // 2
    tab = np.asarray(cos_sin, np.float32)[np.asarray(positions)]     # [N, d]
    c = tab[:, None, :half]
    s = tab[:, None, half:]
    lo, hi = x[..., :half], x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = (lo * c) - (hi * s)          # numpy float32: each op rounded
    out[..., half:] = (hi * c) + (lo * s)
    return out


def rope_quant_append(k_pre, v_new, positions, cos_sin, slot_mapping, k_cache, v_cache,
                      k_scale, v_scale, block_size=BLOCK_SIZE):
    """Rotate K (pre-RoPE bf16 values) at its positions, then quant_append
    the rotated K and the unrotated V."""
    k_rot = rope_rotate_half(k_pre, positions, cos_sin)
    quant_append(k_rot, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, block_size)


# --------------------------------------------------------------------------
# INT4 KV cache.  "KV Cache 优化全景解析" section 2.3 counts INT4 at 0.5 byte
# per element in the KV-size formula, and the KV-cache optimisation page of
# garden.houmin.site (section 2.2.2, directions for optimisation) lists
# compressing the cache from FP16 to INT8 or INT4.
# Readings taken: the INT8 recipe with 7 in place of
# 127, i.e. one fp16 scale per (token, KV head), s = fp16_rne(fp32_rne(
# absmax / 7)), codes = clamp(round_half_even(fp32(x / s)), -7, 7), all zero
# when s == 0; two codes per byte as 4-bit two's complement, element 2i in
# the low nibble of byte i and element 2i+1 in the high nibble; the paged
# layout of the INT8 cache with d/2 bytes per row.
# --------------------------------------------------------------------------
INT4_QMAX = 7


def row_scale_int4(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    s32 = a / np.float32(INT4_QMAX)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    return np.where(np.isinf(s16), np.float16(FP16_MAX), s16).astype(np.float16)


def codes_int4_for_scale(x, s):
    """Signed codes -7..7 (int8 array, unpacked) under fp16 scales s."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = x32 / np.where(zero, np.float32(1), s32)
    q = np.clip(np.rint(quot.astype(np.float64)), -INT4_QMAX, INT4_QMAX)
    return np.where(zero, 0.0, q).astype(np.int8)


def pack_int4(codes):
    """[..., d] signed codes -> [..., d/2] bytes: element 2i in the low
    nibble of byte i, element 2i+1 in the high nibble."""
    c = np.asarray(codes, np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed):
    """[..., d/2] bytes -> [..., d] signed codes (int8)."""
    p = np.asarray(packed, np.int64)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int64)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out.astype(np.int8)


def quantize_rows_int4(x):
    """Rows [..., d] -> (packed codes uint8 [..., d/2], scales fp16 [...])."""
    s = row_scale_int4(x)
    return pack_int4(codes_int4_for_scale(x, s)), s


def dequantize_rows_int4(packed, scales):
    return unpack_int4(packed).astype(np.float64) * \
        np.asarray(scales, np.float16).astype(np.float64)[..., None]


def alloc_paged_cache_int4(num_blocks, num_kv_heads, head_dim, block_size=BLOCK_SIZE):
    kc = np.zeros((num_blocks, num_kv_heads, block_size, head_dim // 2), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((num_blocks, num_kv_heads, block_size), np.float16)
    vs = np.zeros_like(ks)
    return kc, vc, ks, vs


def quant_append_int4(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                      block_size=BLOCK_SIZE):
    """As quant_append, with packed INT4 codes."""
    kc, ks = quantize_rows_int4(k_new)
    vc, vs = quantize_rows_int4(v_new)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = slot_to_block(slot, block_size)
        k_cache[blk, :, off, :] = kc[n]
        v_cache[blk, :, off, :] = vc[n]
        k_scale[blk, :, off] = ks[n]
        v_scale[blk, :, off] = vs[n]


def gather_dequant_int4(packed, scales, block_table_row, ctx, kv_head, block_size=BLOCK_SIZE):
    t = np.arange(ctx)
    blk, off = logical_to_physical(np.asarray(block_table_row), t, block_size)
    return dequantize_rows_int4(packed[blk, kv_head, off, :], scales[blk, kv_head, off])


def paged_decode_int4(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                      sm_scale=None, block_size=BLOCK_SIZE):
    """paged_decode over a packed INT4 cache.  Returns fp64 [B, Hq, d]."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    G = Hq // k_cache.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx <= 0:
            continue
        for h in range(Hq):
            g = kv_head_of(h, G)
            k = gather_dequant_int4(k_cache, k_scale, block_table[b], ctx, g, block_size)
            v = gather_dequant_int4(v_cache, v_scale, block_table[b], ctx, g, block_size)
            out[b, h] = softmax_attention(q[b, h][None, :], k, v, sm_scale)[0]
    return out


def paged_prefill_chunk_int4(q, q_start_loc, k_cache, v_cache, k_scale, v_scale,
                             block_table, context_lens, sm_scale=None, block_size=BLOCK_SIZE):
    """paged_prefill_chunk over a packed INT4 cache.  Returns fp64 [Tq, Hq, d]."""
    q = np.asarray(q, np.float64)
    Tq, Hq, d = q.shape
    G = Hq // k_cache.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((Tq, Hq, d), np.float64)
    for b in range(len(context_lens)):
        r0, r1 = int(q_start_loc[b]), int(q_start_loc[b + 1])
        lc, ctx = r1 - r0, int(context_lens[b])
        if lc <= 0 or ctx <= 0:
            continue
        visible = causal_visibility(ctx, lc)
        for h in range(Hq):
            g = kv_head_of(h, G)
            k = gather_dequant_int4(k_cache, k_scale, block_table[b], ctx, g, block_size)
            v = gather_dequant_int4(v_cache, v_scale, block_table[b], ctx, g, block_size)
            out[r0:r1, h] = softmax_attention(q[r0:r1, h], k, v, sm_scale, visible)
    return out
