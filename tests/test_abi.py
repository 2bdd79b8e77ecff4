"""C ABI checks that need no GPU: the library loads, exports every entry
point include/kv8.h declares, and rejects bad arguments on the host before
any HIP call (so no device is touched)."""
import ctypes
import os
import re

import pytest

from paged_int8_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kv8.h")

# Fake, 16-byte aligned, never dereferenced device addresses
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for st in range(-6, 1):
        assert B.status_string(st).startswith("KV8_")
    assert "unknown" in B.status_string(-99)
    assert B.load().kv8_version() == 200


def append(fn="kv8_quant_append", **kw):
    a = dict(k_new=P, v_new=P, slots=P, n=4, hkv=8, d=128, bs=16, nb=10,
             kc=P, vc=P, ks=P, vs=P, stream=None)
    a.update(kw)
    return getattr(B.load(), fn)(a["k_new"], a["v_new"], a["slots"], a["n"], a["hkv"],
                                     a["d"], a["bs"], a["nb"], a["kc"], a["vc"], a["ks"],
                                     a["vs"], a["stream"])


@pytest.mark.parametrize("kw,expected", [
    (dict(k_new=None), B.KV8_ERR_NULL),
    (dict(slots=None), B.KV8_ERR_NULL),
    (dict(kc=None), B.KV8_ERR_NULL),
    (dict(vs=None), B.KV8_ERR_NULL),
    (dict(n=-1), B.KV8_ERR_SHAPE),
    (dict(hkv=0), B.KV8_ERR_SHAPE),
    (dict(nb=0), B.KV8_ERR_SHAPE),
    (dict(d=96), B.KV8_ERR_UNSUPPORTED),
    (dict(bs=32), B.KV8_ERR_UNSUPPORTED),
    (dict(kc=MIS), B.KV8_ERR_ALIGN),
    (dict(k_new=MIS), B.KV8_ERR_ALIGN),
    (dict(n=0), B.KV8_OK),                      # empty append is a no-op
])
def test_append_validation(kw, expected):
    assert append(**kw) == expected


def decode(fn="paged_decode_attn_kv8", **kw):
    a = dict(q=P, dt=B.KV8_BF16, kc=P, vc=P, ks=P, vs=P, nb=100, bt=P, mbs=16, ctx=P,
             maxctx=256, b=2, hq=32, hkv=8, d=128, bs=16, scale=0.088, out=P, ws=P2,
             wsb=1 << 30, tps=0, form=B.DECODE_AUTO, stream=None)
    a.update(kw)
    return getattr(B.load(), fn)(
        a["q"], a["dt"], a["kc"], a["vc"], a["ks"], a["vs"], a["nb"], a["bt"], a["mbs"],
        a["ctx"], a["maxctx"], a["b"], a["hq"], a["hkv"], a["d"], a["bs"], a["scale"],
        a["out"], a["ws"], a["wsb"], a["tps"], a["form"], a["stream"])


@pytest.mark.parametrize("kw,expected", [
    (dict(q=None), B.KV8_ERR_NULL),
    (dict(bt=None), B.KV8_ERR_NULL),
    (dict(ctx=None), B.KV8_ERR_NULL),
    (dict(out=None), B.KV8_ERR_NULL),
    (dict(ks=None), B.KV8_ERR_NULL),
    (dict(b=0), B.KV8_ERR_SHAPE),
    (dict(hq=30), B.KV8_ERR_SHAPE),             # Hq % Hkv != 0
    (dict(maxctx=-1), B.KV8_ERR_SHAPE),
    (dict(mbs=0), B.KV8_ERR_SHAPE),
    (dict(nb=0), B.KV8_ERR_SHAPE),
    (dict(hq=24), B.KV8_ERR_UNSUPPORTED),       # G = 3
    (dict(d=256), B.KV8_ERR_UNSUPPORTED),
    (dict(bs=32), B.KV8_ERR_UNSUPPORTED),
    (dict(dt=7), B.KV8_ERR_UNSUPPORTED),
    (dict(tps=100), B.KV8_ERR_UNSUPPORTED),
    (dict(tps=4096), B.KV8_ERR_UNSUPPORTED),
    (dict(q=MIS), B.KV8_ERR_ALIGN),
    (dict(kc=MIS), B.KV8_ERR_ALIGN),
    (dict(out=MIS), B.KV8_ERR_ALIGN),
    (dict(ws=None), B.KV8_ERR_WORKSPACE),
    (dict(wsb=16), B.KV8_ERR_WORKSPACE),
    (dict(form=-1), B.KV8_ERR_UNSUPPORTED),
    (dict(form=5), B.KV8_ERR_UNSUPPORTED),
    (dict(b=8193), B.KV8_ERR_SHAPE),            # batch * Hkv above KV8_DECODE_MAX_PAIRS
    (dict(b=8192, ws=None), B.KV8_ERR_WORKSPACE),   # exactly at the limit: accepted
])
def test_decode_validation(kw, expected):
    assert decode(**kw) == expected


@pytest.mark.parametrize("form", [B.DECODE_AUTO, B.DECODE_DOT, B.DECODE_MFMA,
                                  B.DECODE_MFMA_ONEPASS, B.DECODE_STREAMK])
@pytest.mark.parametrize("fn", ["paged_decode_attn_kv8", "paged_decode_attn_fp8kv",
                                "paged_decode_attn_int4kv"])
def test_decode_kernel_form_argument_accepted(fn, form):
    """Every kernel form passes validation (the call then stops at the
    missing workspace, before any HIP call)."""
    assert decode(fn=fn, form=form, ws=None) == B.KV8_ERR_WORKSPACE
    assert decode(fn=fn, form=form + 5) == B.KV8_ERR_UNSUPPORTED


@pytest.mark.parametrize("form,tps,expected", [
    (B.DECODE_DOT, 1280, B.KV8_ERR_WORKSPACE), (B.DECODE_DOT, 1344, B.KV8_ERR_UNSUPPORTED),
    (B.DECODE_MFMA, 1280, B.KV8_ERR_WORKSPACE), (B.DECODE_MFMA, 1344, B.KV8_ERR_UNSUPPORTED),
    (B.DECODE_MFMA_ONEPASS, 2048, B.KV8_ERR_WORKSPACE),
])
def test_decode_split_limit_per_form_at_g8(form, tps, expected):
    """At G = 8 the forms that hold a split's logits in LDS accept at most
    1280 tokens per split; the one-pass form takes up to 2048."""
    assert decode(hq=64, hkv=8, tps=tps, form=form, ws=None) == expected


def test_decode_workspace_counter_region_fixed():
    """The counters occupy a fixed prefix of KV8_DECODE_MAX_PAIRS uint32
    whatever the shape, so a single-split call needs exactly that prefix
    plus its partial arrays, and the limit on pairs is enforced."""
    assert B.MAX_DECODE_PAIRS == 65536
    one = B.kv8_decode_workspace_size(1, 4, 1, 64, 64, 64)
    split_forms = 1024 + 256                 # o (4 heads x 64 fp32) + lse, 256-aligned
    stream_k = 1024 * 2 * (4 * 64 + 2 * 4) * 4   # two states per workgroup, 1024 at most
    assert one == 4 * 65536 + max(split_forms, stream_k)
    assert B.kv8_decode_workspace_size(8193, 8, 8, 128, 64, 0) == 0
    assert B.kv8_decode_workspace_size(8192, 8, 8, 128, 64, 0) > 0


def decode_bf16kv(**kw):
    a = dict(q=P, dt=B.KV8_BF16, kc=P, vc=P, nb=100, bt=P, mbs=16, ctx=P, maxctx=256, b=2,
             hq=32, hkv=8, d=128, bs=16, scale=0.088, out=P, ws=P2, wsb=1 << 30, tps=0,
             stream=None)
    a.update(kw)
    return B.load().paged_decode_attn_bf16kv(
        a["q"], a["dt"], a["kc"], a["vc"], a["nb"], a["bt"], a["mbs"], a["ctx"], a["maxctx"],
        a["b"], a["hq"], a["hkv"], a["d"], a["bs"], a["scale"], a["out"], a["ws"], a["wsb"],
        a["tps"], a["stream"])


@pytest.mark.parametrize("kw,expected", [
    (dict(q=None), B.KV8_ERR_NULL),
    (dict(kc=None), B.KV8_ERR_NULL),
    (dict(vc=None), B.KV8_ERR_NULL),
    (dict(bt=None), B.KV8_ERR_NULL),
    (dict(ctx=None), B.KV8_ERR_NULL),
    (dict(out=None), B.KV8_ERR_NULL),
    (dict(b=0), B.KV8_ERR_SHAPE),
    (dict(hq=30), B.KV8_ERR_SHAPE),
    (dict(maxctx=-1), B.KV8_ERR_SHAPE),
    (dict(mbs=0), B.KV8_ERR_SHAPE),
    (dict(nb=0), B.KV8_ERR_SHAPE),
    (dict(hq=24), B.KV8_ERR_UNSUPPORTED),
    (dict(d=256), B.KV8_ERR_UNSUPPORTED),
    (dict(bs=32), B.KV8_ERR_UNSUPPORTED),
    (dict(dt=7), B.KV8_ERR_UNSUPPORTED),
    (dict(tps=100), B.KV8_ERR_UNSUPPORTED),
    (dict(q=MIS), B.KV8_ERR_ALIGN),
    (dict(vc=MIS), B.KV8_ERR_ALIGN),
    (dict(out=MIS), B.KV8_ERR_ALIGN),
    (dict(ws=None), B.KV8_ERR_WORKSPACE),
    (dict(wsb=16), B.KV8_ERR_WORKSPACE),
])
def test_decode_bf16kv_validation(kw, expected):
    assert decode_bf16kv(**kw) == expected


def test_decode_workspace_size():
    ws = B.kv8_decode_workspace_size(32, 32, 8, 128, 4096, 512)
    n_split = 8
    counters = 4 * B.MAX_DECODE_PAIRS                # fixed counter region
    split_forms = 32 * 32 * n_split * (128 + 1) * 4  # partial outputs and log-sum-exps
    stream_k = 1024 * 2 * (4 * 128 + 2 * 4) * 4      # two states per workgroup, 1024 at most
    assert ws >= counters + max(split_forms, stream_k)
    assert ws < counters + max(split_forms, stream_k) + 512
    assert B.kv8_decode_workspace_size(32, 32, 8, 128, 4096, 0) > 0
    assert B.kv8_decode_workspace_size(32, 30, 8, 128, 4096, 0) == 0
    assert B.kv8_decode_workspace_size(32, 32, 8, 96, 4096, 0) == 0
    assert B.kv8_decode_workspace_size(32, 32, 8, 128, 4096, 100) == 0
    # default split for a Llama-3.1-8B-shaped batch: 1024 tokens
    assert B.kv8_decode_workspace_size(32, 32, 8, 128, 4096, 0) == \
        B.kv8_decode_workspace_size(32, 32, 8, 128, 4096, 1024)


def prefill(fn="paged_prefill_chunk_attn_kv8", **kw):
    a = dict(q=P, qsl=P, tq=64, mq=32, kc=P, vc=P, ks=P, vs=P, nb=100, bt=P, mbs=16, ctx=P,
             maxctx=256, b=2, hq=32, hkv=8, d=128, bs=16, scale=0.088, out=P, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return getattr(B.load(), fn)(
        a["q"], a["qsl"], a["tq"], a["mq"], a["kc"], a["vc"], a["ks"], a["vs"], a["nb"],
        a["bt"], a["mbs"], a["ctx"], a["maxctx"], a["b"], a["hq"], a["hkv"], a["d"], a["bs"],
        a["scale"], a["out"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expected", [
    (dict(qsl=None), B.KV8_ERR_NULL),
    (dict(q=None), B.KV8_ERR_NULL),
    (dict(out=None), B.KV8_ERR_NULL),
    (dict(vc=None), B.KV8_ERR_NULL),
    (dict(b=0), B.KV8_ERR_SHAPE),
    (dict(tq=-1), B.KV8_ERR_SHAPE),
    (dict(hq=31), B.KV8_ERR_SHAPE),
    (dict(hq=48), B.KV8_ERR_UNSUPPORTED),
    (dict(d=80), B.KV8_ERR_UNSUPPORTED),
    (dict(bs=8), B.KV8_ERR_UNSUPPORTED),
    (dict(q=MIS), B.KV8_ERR_ALIGN),
    (dict(ks=MIS), B.KV8_ERR_ALIGN),
    (dict(tq=0), B.KV8_OK),
])
def test_prefill_validation(kw, expected):
    assert prefill(**kw) == expected


@pytest.mark.parametrize("kw", [
    dict(k_new=None), dict(kc=None), dict(vs=None), dict(n=-1), dict(nb=0), dict(d=96),
    dict(bs=32), dict(kc=MIS), dict(n=0),
])
def test_fp8_append_validation_matches_int8(kw):
    assert append(fn="kv8_quant_append_fp8", **kw) == append(**kw)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(ks=None), dict(b=0), dict(hq=30), dict(hq=24), dict(d=256), dict(dt=7),
    dict(tps=100), dict(kc=MIS), dict(ws=None), dict(wsb=16),
])
def test_fp8_decode_validation_matches_int8(kw):
    assert decode(fn="paged_decode_attn_fp8kv", **kw) == decode(**kw)


@pytest.mark.parametrize("kw", [
    dict(qsl=None), dict(vc=None), dict(b=0), dict(tq=-1), dict(hq=31), dict(d=96),
    dict(q=MIS), dict(tq=0),
])
def test_fp8_prefill_validation_matches_int8(kw):
    assert prefill(fn="paged_prefill_chunk_attn_fp8kv", **kw) == prefill(**kw)


def rope_append(**kw):
    a = dict(k_new=P, v_new=P, slots=P, pos=P, cs=P, maxpos=4096, n=4, hkv=8, d=128, bs=16,
             nb=10, kc=P, vc=P, ks=P, vs=P, stream=None)
    a.update(kw)
    return B.load().kv8_rope_quant_append(
        a["k_new"], a["v_new"], a["slots"], a["pos"], a["cs"], a["maxpos"], a["n"], a["hkv"],
        a["d"], a["bs"], a["nb"], a["kc"], a["vc"], a["ks"], a["vs"], a["stream"])


@pytest.mark.parametrize("kw,expected", [
    (dict(pos=None), B.KV8_ERR_NULL),
    (dict(cs=None), B.KV8_ERR_NULL),
    (dict(k_new=None), B.KV8_ERR_NULL),
    (dict(kc=None), B.KV8_ERR_NULL),
    (dict(maxpos=0), B.KV8_ERR_SHAPE),
    (dict(n=-1), B.KV8_ERR_SHAPE),
    (dict(d=96), B.KV8_ERR_UNSUPPORTED),
    (dict(bs=32), B.KV8_ERR_UNSUPPORTED),
    (dict(cs=MIS), B.KV8_ERR_ALIGN),
    (dict(k_new=MIS), B.KV8_ERR_ALIGN),
    (dict(n=0, pos=None, cs=None), B.KV8_OK),
])
def test_rope_append_validation(kw, expected):
    assert rope_append(**kw) == expected


@pytest.mark.parametrize("kw", [
    dict(k_new=None), dict(kc=None), dict(vs=None), dict(n=-1), dict(nb=0), dict(d=96),
    dict(bs=32), dict(kc=MIS), dict(n=0),
])
def test_int4_append_validation_matches_int8(kw):
    assert append(fn="kv8_quant_append_int4", **kw) == append(**kw)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(ks=None), dict(b=0), dict(hq=30), dict(hq=24), dict(d=256), dict(dt=7),
    dict(tps=100), dict(kc=MIS), dict(ws=None), dict(wsb=16),
])
def test_int4_decode_validation_matches_int8(kw):
    assert decode(fn="paged_decode_attn_int4kv", **kw) == decode(**kw)


def test_decode_workspace_covers_every_form():
    """The workspace query sizes for the smallest default split any kernel
    form may take: at G = 8 and 64 sequences of up to 16384 tokens the
    one-pass form takes 2048-token splits and the others 1024, so the query
    answers for 1024 (16 splits)."""
    ws = B.kv8_decode_workspace_size(64, 64, 8, 128, 16384, 0)
    assert ws == B.kv8_decode_workspace_size(64, 64, 8, 128, 16384, 1024)
    assert ws > B.kv8_decode_workspace_size(64, 64, 8, 128, 16384, 2048)


@pytest.mark.parametrize("kw", [
    dict(qsl=None), dict(vc=None), dict(b=0), dict(tq=-1), dict(hq=31), dict(d=96),
    dict(q=MIS), dict(tq=0),
])
def test_int4_prefill_validation_matches_int8(kw):
    assert prefill(fn="paged_prefill_chunk_attn_int4kv", **kw) == prefill(**kw)


def test_read_probe_validation():
    """Host-side checks of the measurement probe: null pointers, tile sizes
    that are not a multiple of 1 KB or exceed 32 KB, byte counts that are
    not whole tiles, workgroup counts out of range, a misaligned buffer."""
    lib = B.load()
    assert lib.kv8_read_probe_chunk_bytes() == 32768
    n = 10 * 32768
    assert lib.kv8_read_probe(None, P, 2048, n, 10, P2, None) == B.KV8_ERR_NULL
    assert lib.kv8_read_probe(P, None, 2048, n, 10, P2, None) == B.KV8_ERR_NULL
    assert lib.kv8_read_probe(P, P, 2048, n, 10, None, None) == B.KV8_ERR_NULL
    for bad in (0, 16, 24, 128, 256, 512, 768, 1536, 3000, 33792, 65536):
        assert lib.kv8_read_probe(P, P, bad, n, 10, P2, None) == B.KV8_ERR_SHAPE
    for bad_n in (0, -2048, 1024, 32768 + 16):
        assert lib.kv8_read_probe(P, P, 2048, bad_n, 10, P2, None) == B.KV8_ERR_SHAPE
    assert lib.kv8_read_probe(P, P, 2048, n, 0, P2, None) == B.KV8_ERR_SHAPE
    assert lib.kv8_read_probe(P, P, 2048, n, 1 << 31, P2, None) == B.KV8_ERR_SHAPE
    assert lib.kv8_read_probe(MIS, P, 2048, n, 10, P2, None) == B.KV8_ERR_ALIGN


def test_stream_read_validation():
    lib = B.load()
    n = 10 * 32768
    assert lib.kv8_stream_read(None, n, 10, P2, None) == B.KV8_ERR_NULL
    assert lib.kv8_stream_read(P, n, 10, None, None) == B.KV8_ERR_NULL
    for bad_n in (0, -32768, 32768 + 16):
        assert lib.kv8_stream_read(P, bad_n, 10, P2, None) == B.KV8_ERR_SHAPE
    assert lib.kv8_stream_read(P, n, 0, P2, None) == B.KV8_ERR_SHAPE
    assert lib.kv8_stream_read(P, n, 1 << 31, P2, None) == B.KV8_ERR_SHAPE
    assert lib.kv8_stream_read(MIS, n, 10, P2, None) == B.KV8_ERR_ALIGN


def decode_noalloc(**kw):
    a = dict(q=P, dt=B.KV8_BF16, kc=P, vc=P, ks=P, vs=P, nb=100, bt=P, mbs=16, ctx=P,
             maxctx=256, b=2, hq=32, hkv=8, d=128, bs=16, scale=0.088, out=P, tps=0,
             form=B.DECODE_AUTO, stream=None)
    a.update(kw)
    return B.load().paged_decode_attn_kv8_noalloc(
        a["q"], a["dt"], a["kc"], a["vc"], a["ks"], a["vs"], a["nb"], a["bt"], a["mbs"],
        a["ctx"], a["maxctx"], a["b"], a["hq"], a["hkv"], a["d"], a["bs"], a["scale"],
        a["out"], a["tps"], a["form"], a["stream"])


@pytest.mark.parametrize("kw,expected", [
    (dict(q=None), B.KV8_ERR_NULL),
    (dict(ks=None), B.KV8_ERR_NULL),
    (dict(b=0), B.KV8_ERR_SHAPE),
    (dict(b=8193), B.KV8_ERR_SHAPE),
    (dict(hq=24), B.KV8_ERR_UNSUPPORTED),
    (dict(form=7), B.KV8_ERR_UNSUPPORTED),
    (dict(tps=100), B.KV8_ERR_UNSUPPORTED),
    (dict(q=MIS), B.KV8_ERR_ALIGN),
    # 64 x 64/8 heads at 65536 tokens in 64-token splits: partials far beyond
    # the fixed scratch, rejected before any HIP call
    (dict(b=64, hq=64, hkv=8, maxctx=65536, mbs=4096, tps=64, form=B.DECODE_MFMA_ONEPASS),
     B.KV8_ERR_WORKSPACE),
])
def test_noalloc_decode_validation(kw, expected):
    """The allocation-free decode validates as paged_decode_attn_kv8 does and
    rejects a call whose partials exceed its fixed scratch, all on the host."""
    assert decode_noalloc(**kw) == expected


def test_noalloc_scratch_covers_the_workloads():
    """The fixed scratch holds the decode workspace of the Llama-3.1-8B-shaped
    batch and of the long-context config under every form, and of a
    Llama-3-70B-shaped layer at the one-pass form's 2048-token splits."""
    cap = B.NOALLOC_SCRATCH_BYTES
    assert B.kv8_decode_workspace_size(32, 32, 8, 128, 4096, 0) <= cap
    assert B.kv8_decode_workspace_size(4, 32, 8, 128, 32768 + 64, 0) <= cap
    assert B.kv8_decode_workspace_size(64, 64, 8, 128, 16384, 2048) <= cap
