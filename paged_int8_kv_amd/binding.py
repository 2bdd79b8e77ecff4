"""ctypes binding of libkv8.so (the C ABI in include/kv8.h).

Argument marshalling only: torch tensors give device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels.  The library must have been built (python -m
paged_int8_kv_amd.build); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

KV8_OK = 0
KV8_ERR_NULL = -1
KV8_ERR_SHAPE = -2
KV8_ERR_UNSUPPORTED = -3
KV8_ERR_ALIGN = -4
KV8_ERR_WORKSPACE = -5
KV8_ERR_HIP = -6
KV8_F32 = 0
KV8_BF16 = 1
BLOCK_SIZE = 16

EXPORTED = (
    "kv8_status_string", "kv8_version", "kv8_quant_append", "kv8_decode_workspace_size",
    "paged_decode_attn_kv8", "paged_decode_attn_bf16kv", "kv8_prefill_workspace_size",
    "paged_prefill_chunk_attn_kv8", "kv8_quant_append_fp8", "paged_decode_attn_fp8kv",
    "paged_prefill_chunk_attn_fp8kv", "kv8_rope_quant_append", "paged_decode_attn_kv8_append",
    "kv8_quant_append_int4", "paged_decode_attn_int4kv",
    "paged_prefill_chunk_attn_int4kv", "kv8_read_probe_chunk_bytes", "kv8_read_probe",
    "kv8_stream_read", "paged_decode_attn_kv8_noalloc",
)

_lib = None


class Kv8Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def lib_path():
    return _build.LIB_PATH


def load():
    """Load libkv8.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libkv8.so not built at {path}; run python -m paged_int8_kv_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.kv8_status_string.restype = ctypes.c_char_p
    lib.kv8_status_string.argtypes = [i32]
    lib.kv8_version.restype = i32
    lib.kv8_version.argtypes = []
    lib.kv8_quant_append.restype = i32
    lib.kv8_quant_append.argtypes = [vp, vp, vp, i64, i32, i32, i32, i64, vp, vp, vp, vp, vp]
    lib.kv8_rope_quant_append.restype = i32
    lib.kv8_rope_quant_append.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i64,
                                          vp, vp, vp, vp, vp]
    lib.kv8_quant_append_fp8.restype = i32
    lib.kv8_quant_append_fp8.argtypes = lib.kv8_quant_append.argtypes
    lib.kv8_quant_append_int4.restype = i32
    lib.kv8_quant_append_int4.argtypes = lib.kv8_quant_append.argtypes
    lib.kv8_decode_workspace_size.restype = sz
    lib.kv8_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.paged_decode_attn_kv8.restype = i32
    lib.paged_decode_attn_kv8.argtypes = [vp, i32, vp, vp, vp, vp, i64, vp, i32, vp, i32,
                                          i32, i32, i32, i32, i32, f32, vp, vp, sz, i32, i32,
                                          vp]
    lib.paged_decode_attn_kv8_noalloc.restype = i32
    lib.paged_decode_attn_kv8_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, i64, vp, i32, vp,
                                                  i32, i32, i32, i32, i32, i32, f32, vp, i32,
                                                  i32, vp]
    lib.paged_decode_attn_kv8_append.restype = i32
    lib.paged_decode_attn_kv8_append.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i64, vp, i32,
                                                 vp, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                                 sz, i32, i32, vp]
    lib.paged_decode_attn_fp8kv.restype = i32
    lib.paged_decode_attn_fp8kv.argtypes = lib.paged_decode_attn_kv8.argtypes
    lib.paged_decode_attn_int4kv.restype = i32
    lib.paged_decode_attn_int4kv.argtypes = lib.paged_decode_attn_kv8.argtypes
    lib.paged_decode_attn_bf16kv.restype = i32
    lib.paged_decode_attn_bf16kv.argtypes = [vp, i32, vp, vp, i64, vp, i32, vp, i32,
                                             i32, i32, i32, i32, i32, f32, vp, vp, sz, i32, vp]
    lib.kv8_prefill_workspace_size.restype = sz
    lib.kv8_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.paged_prefill_chunk_attn_kv8.restype = i32
    lib.paged_prefill_chunk_attn_kv8.argtypes = [vp, vp, i64, i32, vp, vp, vp, vp, i64, vp,
                                                 i32, vp, i32, i32, i32, i32, i32, i32, f32,
                                                 vp, vp, sz, vp]
    lib.paged_prefill_chunk_attn_fp8kv.restype = i32
    lib.paged_prefill_chunk_attn_fp8kv.argtypes = lib.paged_prefill_chunk_attn_kv8.argtypes
    lib.kv8_read_probe_chunk_bytes.restype = i64
    lib.kv8_read_probe_chunk_bytes.argtypes = []
    lib.kv8_read_probe.restype = i32
    lib.kv8_read_probe.argtypes = [vp, vp, i32, i64, i64, vp, vp]
    lib.kv8_stream_read.restype = i32
    lib.kv8_stream_read.argtypes = [vp, i64, i64, vp, vp]
    lib.paged_prefill_chunk_attn_int4kv.restype = i32
    lib.paged_prefill_chunk_attn_int4kv.argtypes = lib.paged_prefill_chunk_attn_kv8.argtypes
    _lib = lib
    return lib


# decode kernel forms (the kernel_form argument of the INT8 / FP8 / INT4
# decode calls): automatic, v_dot2, two-pass matrix-core, one-pass
# matrix-core, stream-K matrix-core
DECODE_AUTO, DECODE_DOT, DECODE_MFMA, DECODE_MFMA_ONEPASS, DECODE_STREAMK = 0, 1, 2, 3, 4
MAX_DECODE_PAIRS = 65536


def status_string(status):
    return load().kv8_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, where):
    if status != KV8_OK:
        raise Kv8Error(status, where)


# ---------------------------------------------------------------------------
# torch-facing wrappers (same names as the C entry points)
# ---------------------------------------------------------------------------
def _append(name, k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream):
    n, hkv, d = k_new.shape
    nb = k_cache.shape[0]
    st = getattr(load(), name)(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), n, hkv, d,
                               BLOCK_SIZE, nb, _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                               _ptr(v_scale), _stream(stream))
    _check(st, name)


def kv8_quant_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                     stream=None):
    """k_new/v_new: bf16 [N, Hkv, d]; slot_mapping int32 [N]; caches as in
    include/kv8.h.  Enqueues on the current (or given) stream."""
    _append("kv8_quant_append", k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
            stream)


def kv8_quant_append_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                         stream=None):
    """As kv8_quant_append, into an FP8 (e4m3) cache (uint8 codes)."""
    _append("kv8_quant_append_fp8", k_new, v_new, slot_mapping, k_cache, v_cache, k_scale,
            v_scale, stream)


def kv8_rope_quant_append(k_new, v_new, slot_mapping, positions, cos_sin, k_cache, v_cache,
                          k_scale, v_scale, stream=None):
    """k_new (before RoPE) / v_new: bf16 [N, Hkv, d]; slot_mapping and
    positions int32 [N]; cos_sin fp32 [max_position, d]."""
    n, hkv, d = k_new.shape
    st = load().kv8_rope_quant_append(
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], n, hkv, d, BLOCK_SIZE, k_cache.shape[0], _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _stream(stream))
    _check(st, "kv8_rope_quant_append")


def kv8_quant_append_int4(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                          stream=None):
    """As kv8_quant_append, into an INT4 cache (packed codes uint8
    [NB, Hkv, 16, d/2])."""
    _append("kv8_quant_append_int4", k_new, v_new, slot_mapping, k_cache, v_cache, k_scale,
            v_scale, stream)


def kv8_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_context_len,
                              tokens_per_split=0):
    return int(load().kv8_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, tokens_per_split))


def _decode(name, q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
            max_context_len, out, workspace, sm_scale, tokens_per_split, kernel_form, stream):
    import torch
    b, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    dt = KV8_BF16 if q.dtype == torch.bfloat16 else KV8_F32
    if sm_scale is None:
        sm_scale = d ** -0.5
    st = getattr(load(), name)(
        _ptr(q), dt, _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), nb,
        _ptr(block_table), block_table.shape[1], _ptr(context_lens), int(max_context_len),
        b, hq, hkv, d, BLOCK_SIZE, float(sm_scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        int(tokens_per_split), int(kernel_form), _stream(stream))
    _check(st, name)


def paged_decode_attn_kv8(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                          max_context_len, out, workspace, sm_scale=None, tokens_per_split=0,
                          kernel_form=DECODE_AUTO, stream=None):
    """q: fp32 or bf16 [B, Hq, d]; out fp32 [B, Hq, d]; workspace uint8 of at
    least kv8_decode_workspace_size() bytes; kernel_form one of DECODE_*."""
    _decode("paged_decode_attn_kv8", q, k_cache, v_cache, k_scale, v_scale, block_table,
            context_lens, max_context_len, out, workspace, sm_scale, tokens_per_split,
            kernel_form, stream)


NOALLOC_SCRATCH_BYTES = 32 << 20


def paged_decode_attn_kv8_noalloc(q, k_cache, v_cache, k_scale, v_scale, block_table,
                                  context_lens, max_context_len, out, sm_scale=None,
                                  tokens_per_split=0, kernel_form=DECODE_AUTO, stream=None):
    """As paged_decode_attn_kv8 with the library's fixed scratch in place of
    a workspace: allocates nothing (calls that overlap on one device race)."""
    import torch
    b, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    dt = KV8_BF16 if q.dtype == torch.bfloat16 else KV8_F32
    if sm_scale is None:
        sm_scale = d ** -0.5
    st = load().paged_decode_attn_kv8_noalloc(
        _ptr(q), dt, _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), nb,
        _ptr(block_table), block_table.shape[1], _ptr(context_lens), int(max_context_len),
        b, hq, hkv, d, BLOCK_SIZE, float(sm_scale), _ptr(out), int(tokens_per_split),
        int(kernel_form), _stream(stream))
    _check(st, "paged_decode_attn_kv8_noalloc")


def paged_decode_attn_int4kv(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                             max_context_len, out, workspace, sm_scale=None, tokens_per_split=0,
                             kernel_form=DECODE_AUTO, stream=None):
    """As paged_decode_attn_kv8, over an INT4 cache."""
    _decode("paged_decode_attn_int4kv", q, k_cache, v_cache, k_scale, v_scale, block_table,
            context_lens, max_context_len, out, workspace, sm_scale, tokens_per_split,
            kernel_form, stream)


def paged_decode_attn_fp8kv(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                            max_context_len, out, workspace, sm_scale=None, tokens_per_split=0,
                            kernel_form=DECODE_AUTO, stream=None):
    """As paged_decode_attn_kv8, over an FP8 (e4m3) cache."""
    _decode("paged_decode_attn_fp8kv", q, k_cache, v_cache, k_scale, v_scale, block_table,
            context_lens, max_context_len, out, workspace, sm_scale, tokens_per_split,
            kernel_form, stream)


def paged_decode_attn_kv8_append(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                 block_table, context_lens, max_context_len, out, workspace,
                                 sm_scale=None, tokens_per_split=0, kernel_form=DECODE_AUTO,
                                 stream=None):
    """One decode step: append k_new/v_new (bf16 [B, Hkv, d], the newest token
    of each sequence, at position context_lens[b] - 1), then decode."""
    import torch
    b, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    dt = KV8_BF16 if q.dtype == torch.bfloat16 else KV8_F32
    if sm_scale is None:
        sm_scale = d ** -0.5
    st = load().paged_decode_attn_kv8_append(
        _ptr(q), dt, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), nb, _ptr(block_table), block_table.shape[1], _ptr(context_lens),
        int(max_context_len), b, hq, hkv, d, BLOCK_SIZE, float(sm_scale), _ptr(out),
        _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        int(tokens_per_split), int(kernel_form), _stream(stream))
    _check(st, "paged_decode_attn_kv8_append")


def paged_decode_attn_bf16kv(q, k_cache, v_cache, block_table, context_lens, max_context_len,
                             out, workspace, sm_scale=None, tokens_per_split=0, stream=None):
    """Decode over a paged bf16 cache.  q: fp32 or bf16 [B, Hq, d]; k_cache,
    v_cache: bf16 (or int16 holding bf16 bits) [NB, Hkv, 16, d]; out fp32
    [B, Hq, d]; workspace uint8 of at least kv8_decode_workspace_size()
    bytes."""
    import torch
    b, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    dt = KV8_BF16 if q.dtype == torch.bfloat16 else KV8_F32
    if sm_scale is None:
        sm_scale = d ** -0.5
    st = load().paged_decode_attn_bf16kv(
        _ptr(q), dt, _ptr(k_cache), _ptr(v_cache), nb, _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), int(max_context_len), b, hq, hkv, d, BLOCK_SIZE, float(sm_scale),
        _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        int(tokens_per_split), _stream(stream))
    _check(st, "paged_decode_attn_bf16kv")


def kv8_prefill_workspace_size(batch, num_q_heads, head_dim, max_q_len, max_context_len):
    return int(load().kv8_prefill_workspace_size(batch, num_q_heads, head_dim, max_q_len,
                                                 max_context_len))


def _prefill(name, q, q_start_loc, max_q_len, k_cache, v_cache, k_scale, v_scale, block_table,
             context_lens, max_context_len, out, workspace, sm_scale, stream):
    tq, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    b = context_lens.shape[0]
    if sm_scale is None:
        sm_scale = d ** -0.5
    st = getattr(load(), name)(
        _ptr(q), _ptr(q_start_loc), tq, int(max_q_len), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), nb, _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), int(max_context_len), b, hq, hkv, d, BLOCK_SIZE, float(sm_scale),
        _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check(st, name)


def paged_prefill_chunk_attn_kv8(q, q_start_loc, max_q_len, k_cache, v_cache, k_scale, v_scale,
                                 block_table, context_lens, max_context_len, out,
                                 workspace=None, sm_scale=None, stream=None):
    """q: bf16 [total_q, Hq, d]; q_start_loc int32 [B+1]; out fp32
    [total_q, Hq, d]."""
    _prefill("paged_prefill_chunk_attn_kv8", q, q_start_loc, max_q_len, k_cache, v_cache,
             k_scale, v_scale, block_table, context_lens, max_context_len, out, workspace,
             sm_scale, stream)


def paged_prefill_chunk_attn_fp8kv(q, q_start_loc, max_q_len, k_cache, v_cache, k_scale,
                                   v_scale, block_table, context_lens, max_context_len, out,
                                   workspace=None, sm_scale=None, stream=None):
    """As paged_prefill_chunk_attn_kv8, over an FP8 (e4m3) cache."""
    _prefill("paged_prefill_chunk_attn_fp8kv", q, q_start_loc, max_q_len, k_cache, v_cache,
             k_scale, v_scale, block_table, context_lens, max_context_len, out, workspace,
             sm_scale, stream)


def paged_prefill_chunk_attn_int4kv(q, q_start_loc, max_q_len, k_cache, v_cache, k_scale,
                                    v_scale, block_table, context_lens, max_context_len, out,
                                    workspace=None, sm_scale=None, stream=None):
    """As paged_prefill_chunk_attn_kv8, over an INT4 (nibble-packed) cache."""
    _prefill("paged_prefill_chunk_attn_int4kv", q, q_start_loc, max_q_len, k_cache, v_cache,
             k_scale, v_scale, block_table, context_lens, max_context_len, out, workspace,
             sm_scale, stream)


def kv8_read_probe(buf, tiles, tile_bytes, workgroups, out, stream=None):
    """Measurement utility: one launch of the random-tile read over `buf`
    (uint8 device tensor) in the tile order `tiles` (int32, tiles of
    tile_bytes, a multiple of 1024 up to 32768) by `workgroups` persistent
    workgroups; `out` uint32 [workgroups * 256].  Returns the bytes the
    launch reads."""
    n_bytes = tiles.numel() * tile_bytes
    if workgroups * 256 > out.numel():
        raise ValueError("out too small")
    _check(load().kv8_read_probe(_ptr(buf), _ptr(tiles), int(tile_bytes), int(n_bytes),
                                 int(workgroups), _ptr(out), _stream(stream)), "kv8_read_probe")
    return n_bytes


def kv8_stream_read(buf, workgroups, out, stream=None):
    """Measurement utility: one launch of the contiguous streaming read over
    the whole of `buf` (uint8 device tensor, size a multiple of the chunk
    size) by `workgroups` persistent workgroups; `out` uint32
    [workgroups * 256].  Returns the bytes the launch reads."""
    if workgroups * 256 > out.numel():
        raise ValueError("out too small")
    _check(load().kv8_stream_read(_ptr(buf), int(buf.numel()), int(workgroups), _ptr(out),
                                  _stream(stream)), "kv8_stream_read")
    return int(buf.numel())


def alloc_cache(num_blocks, num_kv_heads, head_dim, device="cuda", fp8=False, int4=False):
    """Zeroed paged cache tensors: codes int8 [NB, Hkv, 16, d] (uint8 for the
    FP8 cache; uint8 [NB, Hkv, 16, d/2] of packed nibbles for the INT4 cache)
    and fp16 scales [NB, Hkv, 16] (stored as int16 bit patterns), for K and
    V."""
    import torch
    kc = torch.zeros((num_blocks, num_kv_heads, BLOCK_SIZE, head_dim // 2 if int4 else head_dim),
                     dtype=torch.uint8 if (fp8 or int4) else torch.int8, device=device)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((num_blocks, num_kv_heads, BLOCK_SIZE), dtype=torch.int16, device=device)
    vs = torch.zeros_like(ks)
    return kc, vc, ks, vs
