"""Planted mistakes in the oracle must be caught by its pins.

Each mutant swaps one oracle helper for a copy carrying one plausible slip
(a wrong index, a dropped term, a transposed operand, a wrong rounding or
clamp).  The pin battery from test_oracle_pins must then fail.  CPU only;
the mutation lives in the oracle process, never on a GPU.
"""
import numpy as np
import pytest

import tests.test_oracle_pins as P
from oracle import kv8_oracle as O


def _battery():
    """Run the pins, cheapest first; return the name of the first failing
    one, or None if all pass."""
    checks = [
        ("ties_clamp", P.test_quantiser_ties_to_even_and_clamp),
        ("invariants", P.test_quantiser_invariants),
        ("append", P.test_append_scatter_and_skip),
        ("brute_force", P.test_decode_brute_force_tiny),
        ("closed_forms", P.test_decode_closed_forms),
        ("dominant_key", P.test_decode_dominant_key_large_logits),
        ("sdpa_gqa", lambda: P.test_decode_matches_sdpa_fp64(
            lambda: P.W.make_paged_case(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=32,
                                        context_lens=[1, 17, 300], q_dtype="bf16",
                                        k_outliers=True, seed=4))),
        ("prefill_causal", P.test_prefill_no_context_equals_sdpa_causal),
        ("prefill_ctx", P.test_prefill_with_context_equals_sdpa_masked_and_locality),
        ("page_example", P.test_block_table_example_from_page),
        ("scale_exhaustive", P.test_scale_exhaustive_all_bf16_absmax),
        ("kv_size", P.test_kv_size_printed_tables),
        ("bf16_brute_force", P.test_bf16_decode_brute_force_tiny),
        ("bf16_sdpa", P.test_bf16_decode_matches_sdpa_fp64),
        ("bf16_closed_forms", P.test_bf16_decode_closed_forms_and_permutation),
        ("bf16_vs_int8", P.test_bf16_decode_equals_int8_decode_on_exact_values),
        ("fp8_decode_codes", P.test_fp8_decode_every_code_vs_torch),
        ("fp8_encode", P.test_fp8_encode_every_bf16_vs_torch_and_saturation),
        ("fp8_quantiser", P.test_fp8_quantiser_invariants),
        ("fp8_decode", P.test_fp8_decode_brute_force_and_sdpa),
        ("fp8_prefill", P.test_fp8_prefill_equals_sdpa_causal),
        ("rope_library", P.test_rope_matches_transformers_and_fp64),
        ("rope_props", P.test_rope_identity_at_zero_and_relative_position),
        ("rope_append", P.test_rope_quant_append_is_rotate_then_quantise),
        ("int4_pack", P.test_int4_packing_worked_example_and_roundtrip),
        ("int4_invariants", P.test_int4_quantiser_invariants),
        ("int4_attention", P.test_int4_decode_and_prefill_brute_force),
        ("int4_codes", lambda: P.test_int4_codes_every_bf16(1.0)),
        ("int4_scale_exhaustive", P.test_int4_scale_every_bf16_absmax),
        ("codes_exhaustive", lambda: [P.test_codes_exhaustive_all_bf16(s) for s in P.SCALES]),
        ("fp8_scale_exhaustive", P.test_fp8_scale_every_bf16_absmax),
        ("fp8_codes_exhaustive", lambda: [P.test_fp8_codes_every_bf16(s) for s in P.FP8_SCALES]),
    ]
    for name, fn in checks:
        try:
            fn()
        except Exception:          # an assertion or a numerical blow-up
            return name
    return None


def _softmax_no_scale(q_rows, k, v, sm_scale, visible=None):
    scores = q_rows @ k.T
    if visible is not None:
        scores = np.where(visible, scores, -np.inf)
    m = np.max(scores, axis=-1, keepdims=True)
    p = np.exp(scores - m)
    return (p @ v) / np.sum(p, axis=-1, keepdims=True)


def _softmax_no_max(q_rows, k, v, sm_scale, visible=None):
    scores = (q_rows @ k.T) * sm_scale
    if visible is not None:
        scores = np.where(visible, scores, -np.inf)
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(scores)
        return (p @ v) / np.sum(p, axis=-1, keepdims=True)


def _softmax_transposed_v(q_rows, k, v, sm_scale, visible=None):
    scores = (q_rows @ k.T) * sm_scale
    if visible is not None:
        scores = np.where(visible, scores, -np.inf)
    m = np.max(scores, axis=-1, keepdims=True)
    p = np.exp(scores - m)
    w = p / np.sum(p, axis=-1, keepdims=True)
    return (w @ k)          # multiplies by K instead of V


def _row_scale_128(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = (a / np.float32(128)).astype(np.float16)
    return np.where(np.isinf(s16), np.float16(65504), s16).astype(np.float16)


def _row_scale_mean(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.mean(np.abs(x), axis=-1).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = (a / np.float32(127)).astype(np.float16)
    return np.where(np.isinf(s16), np.float16(65504), s16).astype(np.float16)


def _codes_half_away(x, s):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = (x32 / np.where(zero, np.float32(1), s32)).astype(np.float64)
    q = np.sign(quot) * np.floor(np.abs(quot) + 0.5)
    q = np.where(zero, 0.0, np.clip(q, -127, 127))
    return q.astype(np.int8)


def _codes_clamp_128(x, s):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = (x32 / np.where(zero, np.float32(1), s32)).astype(np.float64)
    q = np.where(zero, 0.0, np.clip(np.rint(quot), -128, 127))
    return q.astype(np.int8)


def _codes_truncate(x, s):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = (x32 / np.where(zero, np.float32(1), s32)).astype(np.float64)
    q = np.where(zero, 0.0, np.clip(np.trunc(quot), -127, 127))
    return q.astype(np.int8)


def _dequant_sign_flip(codes, scales):
    return -codes.astype(np.float64) * np.asarray(scales, np.float16).astype(np.float64)[..., None]


def _bf16_as_fp16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _bf16_low_half(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(8)
    return b.view(np.float32).astype(np.float64)


def _gather_bf16_head0(cache_bits, block_table_row, ctx, kv_head, block_size=16):
    t = np.arange(ctx)
    blk, off = np.asarray(block_table_row)[t // block_size], t % block_size
    return O.bf16_bits_to_f64(cache_bits[blk, 0, off, :])


def _e4m3_truncate(x):
    x = np.asarray(x, np.float32).astype(np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)
    ulp = np.exp2(e - 3)
    r = np.minimum(np.floor(a / ulp) * ulp, 448.0)
    sub = r < 2.0 ** -6
    ee = np.where(sub, 0, np.floor(np.log2(np.where(sub, 1.0, r))) + 7).astype(np.int64)
    mm = np.where(sub, np.rint(r / 2.0 ** -9),
                  np.rint(r / np.exp2(ee.astype(np.float64) - 7) * 8) - 8).astype(np.int64)
    return (np.where(np.signbit(x), 0x80, 0) | (ee << 3) | mm).astype(np.uint8)


def _e4m3_value_bias8(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -10, (8 + m) * np.exp2(e.astype(np.float64) - 11))
    return sign * np.where((c & 0x7F) == 0x7F, np.nan, mag)


def _row_scale_fp8_127(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = (a / np.float32(127)).astype(np.float16)
    return np.where(np.isinf(s16), np.float16(65504), s16).astype(np.float16)


def _fp16_truncate(s32):
    """fp32 -> fp16 rounding toward zero (a plausible slip for RNE)."""
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    over = np.abs(s16.astype(np.float32)) > np.abs(s32)
    return np.where(over, np.nextafter(s16, np.float16(0)), s16).astype(np.float16)


def _row_scale_fp8_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    s16 = _fp16_truncate(a / np.float32(448))
    return np.where(np.isinf(s16), np.float16(65504), s16).astype(np.float16)


def _row_scale_fp8_no_saturation(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    with np.errstate(over="ignore"):
        return (a / np.float32(448)).astype(np.float16)


def _codes_fp8_quotient_fp16(x, s):
    x16 = np.asarray(x, dtype=np.float64).astype(np.float16)
    s16 = np.asarray(s, dtype=np.float16)[..., None]
    zero = s16 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = x16 / np.where(zero, np.float16(1), s16)
    return np.where(zero, np.uint8(0), O.e4m3_encode(quot.astype(np.float32))).astype(np.uint8)


def _codes_fp8_reciprocal(x, s):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = x32 * (np.float32(1) / np.where(zero, np.float32(1), s32))
    return np.where(zero, np.uint8(0), O.e4m3_encode(quot)).astype(np.uint8)


def _codes_reciprocal(x, s):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = x32 * (np.float32(1) / np.where(zero, np.float32(1), s32))
    q = np.where(zero, 0.0, np.clip(np.rint(quot.astype(np.float64)), -127, 127))
    return q.astype(np.int8)


def _row_scale_int4_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    s16 = _fp16_truncate(a / np.float32(7))
    return np.where(np.isinf(s16), np.float16(65504), s16).astype(np.float16)


def _rope_sign(x, positions, cos_sin):
    x = np.asarray(x, np.float32)
    half = x.shape[-1] // 2
    tab = np.asarray(cos_sin, np.float32)[np.asarray(positions)]
    c, s_ = tab[:, None, :half], tab[:, None, half:]
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c + hi * s_, hi * c - lo * s_], axis=-1)


def _rope_cos_sin_swapped(x, positions, cos_sin):
    x = np.asarray(x, np.float32)
    half = x.shape[-1] // 2
    tab = np.asarray(cos_sin, np.float32)[np.asarray(positions)]
    s_, c = tab[:, None, :half], tab[:, None, half:]
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s_, hi * c + lo * s_], axis=-1)


def _rope_interleaved(x, positions, cos_sin):
    x = np.asarray(x, np.float32)
    half = x.shape[-1] // 2
    tab = np.asarray(cos_sin, np.float32)[np.asarray(positions)]
    c, s_ = tab[:, None, :half], tab[:, None, half:]
    ev, od = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = ev * c - od * s_
    out[..., 1::2] = od * c + ev * s_
    return out


def _pack_int4_swapped(codes):
    c = np.asarray(codes, np.int64) & 0xF
    return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)


def _row_scale_int4_8(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.max(np.abs(x), axis=-1).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = (a / np.float32(8)).astype(np.float16)
    return np.where(np.isinf(s16), np.float16(65504), s16).astype(np.float16)


def _unpack_int4_sign_magnitude(packed):
    p = np.asarray(packed, np.int64)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int64)
    out[..., 0::2] = np.where(lo >= 8, -(lo - 8), lo)
    out[..., 1::2] = np.where(hi >= 8, -(hi - 8), hi)
    return out.astype(np.int8)


def _gather_scale_of_head0(codes, scales, block_table_row, ctx, kv_head, block_size=16):
    t = np.arange(ctx)
    blk, off = O.logical_to_physical(np.asarray(block_table_row), t, block_size)
    return O.dequantize_rows(codes[blk, kv_head, off, :], scales[blk, 0, off])   # head 0's scales


def _gather_scale_next_token(codes, scales, block_table_row, ctx, kv_head, block_size=16):
    t = np.arange(ctx)
    blk, off = O.logical_to_physical(np.asarray(block_table_row), t, block_size)
    return O.dequantize_rows(codes[blk, kv_head, off, :],
                             scales[blk, kv_head, (off + 1) % block_size])


def _append_no_skip(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                    block_size=16):
    kc, ks = O.quantize_rows(k_new)
    vc, vs = O.quantize_rows(v_new)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):   # negative slots written too
        blk, off = O.slot_to_block(slot, block_size)
        k_cache[blk, :, off, :] = kc[n]
        v_cache[blk, :, off, :] = vc[n]
        k_scale[blk, :, off] = ks[n]
        v_scale[blk, :, off] = vs[n]


def _decode_drops_newest(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                         sm_scale=None, block_size=16):
    return _REAL["paged_decode"](q, k_cache, v_cache, k_scale, v_scale, block_table,
                                 np.maximum(np.asarray(context_lens) - 1, 0), sm_scale, block_size)


def _prefill_rows_from_zero(q, q_start_loc, k_cache, v_cache, k_scale, v_scale, block_table,
                            context_lens, sm_scale=None, block_size=16):
    qs = np.asarray(q_start_loc).copy()
    lens = np.diff(qs)
    out = np.zeros(np.asarray(q).shape, np.float64)
    for b in range(len(lens)):      # every sequence's rows read from row 0
        one = _REAL["paged_prefill_chunk"](np.asarray(q)[:lens[b]], np.array([0, lens[b]]),
                                           k_cache, v_cache, k_scale, v_scale,
                                           np.asarray(block_table)[b:b + 1],
                                           np.asarray(context_lens)[b:b + 1], sm_scale, block_size)
        out[qs[b]:qs[b + 1]] = one
    return out


def _int4_codes_clamp_8(x, s):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = x32 / np.where(zero, np.float32(1), s32)
    q = np.clip(np.rint(quot.astype(np.float64)), -8, 7)
    return np.where(zero, 0.0, q).astype(np.int8)


def _int4_codes_half_away(x, s):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)[..., None]
    zero = s32 == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quot = (x32 / np.where(zero, np.float32(1), s32)).astype(np.float64)
    q = np.clip(np.sign(quot) * np.floor(np.abs(quot) + 0.5), -7, 7)
    return np.where(zero, 0.0, q).astype(np.int8)


def _fp8_dequant_no_scale(codes, scales):
    return O.e4m3_value(codes) + 0.0 * np.asarray(scales, np.float16).astype(np.float64)[..., None]


def _int4_dequant_no_scale(packed, scales):
    return O.unpack_int4(packed).astype(np.float64) + \
        0.0 * np.asarray(scales, np.float16).astype(np.float64)[..., None]


def _rope_append_position_plus_one(k_pre, v_new, positions, cos_sin, slot_mapping, k_cache,
                                   v_cache, k_scale, v_scale, block_size=16):
    k_rot = O.rope_rotate_half(k_pre, np.asarray(positions) + 1, cos_sin)
    O.quant_append(k_rot, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, block_size)


_REAL = {"paged_decode": O.paged_decode, "paged_prefill_chunk": O.paged_prefill_chunk}


MUTANTS = {
    "gather_scale_of_head0": ("gather_dequant", _gather_scale_of_head0),
    "gather_scale_next_token": ("gather_dequant", _gather_scale_next_token),
    "append_no_skip": ("quant_append", _append_no_skip),
    "decode_drops_newest": ("paged_decode", _decode_drops_newest),
    "prefill_rows_from_zero": ("paged_prefill_chunk", _prefill_rows_from_zero),
    "int4_codes_clamp_8": ("codes_int4_for_scale", _int4_codes_clamp_8),
    "int4_codes_half_away": ("codes_int4_for_scale", _int4_codes_half_away),
    "fp8_dequant_no_scale": ("dequantize_rows_fp8", _fp8_dequant_no_scale),
    "int4_dequant_no_scale": ("dequantize_rows_int4", _int4_dequant_no_scale),
    "rope_append_position_plus_one": ("rope_quant_append", _rope_append_position_plus_one),
    "head_map_mod": ("kv_head_of", lambda h, group: h % group),
    "page_transposed": ("logical_to_physical", lambda row, t, bs=16: (row[t % bs], t // bs)),
    "page_identity": ("logical_to_physical", lambda row, t, bs=16: (t // bs, t % bs)),
    "slot_swapped": ("slot_to_block", lambda slot, bs=16: (slot % bs, slot // bs)),
    "softmax_no_scale": ("softmax_attention", _softmax_no_scale),
    "softmax_no_max": ("softmax_attention", _softmax_no_max),
    "softmax_times_k": ("softmax_attention", _softmax_transposed_v),
    "scale_div_128": ("row_scale", _row_scale_128),
    "scale_mean": ("row_scale", _row_scale_mean),
    "codes_half_away": ("codes_for_scale", _codes_half_away),
    "codes_clamp_128": ("codes_for_scale", _codes_clamp_128),
    "codes_truncate": ("codes_for_scale", _codes_truncate),
    "codes_reciprocal": ("codes_for_scale", _codes_reciprocal),
    "dequant_sign": ("dequantize_rows", _dequant_sign_flip),
    "causal_exclusive": ("causal_visibility",
                         lambda ctx, lc: np.arange(ctx)[None, :] < (ctx - lc + np.arange(lc))[:, None]),
    "causal_off_by_one": ("causal_visibility",
                          lambda ctx, lc: np.arange(ctx)[None, :] <= (ctx - lc + 1 + np.arange(lc))[:, None]),
    "kv_size_no_two": ("kv_cache_bytes", lambda L, B, T, H, d, nb: L * B * T * H * d * nb),
    "bf16_read_as_fp16": ("bf16_bits_to_f64", _bf16_as_fp16),
    "bf16_wrong_shift": ("bf16_bits_to_f64", _bf16_low_half),
    "bf16_gather_head0": ("gather_bf16", _gather_bf16_head0),
    "fp8_encode_truncates": ("e4m3_encode", _e4m3_truncate),
    "fp8_value_bias8": ("e4m3_value", _e4m3_value_bias8),
    "fp8_scale_127": ("row_scale_fp8", _row_scale_fp8_127),
    "fp8_scale_truncates": ("row_scale_fp8", _row_scale_fp8_truncate),
    "fp8_scale_no_saturation": ("row_scale_fp8", _row_scale_fp8_no_saturation),
    "fp8_quotient_fp16": ("codes_fp8_for_scale", _codes_fp8_quotient_fp16),
    "fp8_quotient_reciprocal": ("codes_fp8_for_scale", _codes_fp8_reciprocal),
    "int4_scale_truncates": ("row_scale_int4", _row_scale_int4_truncate),
    "rope_sign": ("rope_rotate_half", _rope_sign),
    "rope_cos_sin_swapped": ("rope_rotate_half", _rope_cos_sin_swapped),
    "rope_interleaved": ("rope_rotate_half", _rope_interleaved),
    "int4_nibbles_swapped": ("pack_int4", _pack_int4_swapped),
    "int4_scale_8": ("row_scale_int4", _row_scale_int4_8),
    "int4_sign_magnitude": ("unpack_int4", _unpack_int4_sign_magnitude),
}


def test_unmutated_battery_passes():
    assert _battery() is None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, repl = MUTANTS[name]
    monkeypatch.setattr(O, attr, repl)
    caught = _battery()
    assert caught is not None, f"mutant {name} passed every pin"
