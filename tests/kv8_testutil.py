"""Shared helpers of the GPU parity tests: moving seeded cases to the
device, building caches on either side, and the tolerance check."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B

# Attention tolerance: max |delta| <= 2e-3 and ||delta||_2 / ||ref||_2 <= 1e-3,
# evaluated in fp32 against the fp64 oracle on the same dequantised cache.
MAX_ABS = 2e-3
REL_L2 = 1e-3

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")

# Decode kernel form the helpers pass to every decode call (the
# decode_kernel fixture sets it per test; the library keeps no setting).
FORM = B.DECODE_AUTO


def form(kernel_form=None):
    return FORM if kernel_form is None else kernel_form


def dev():
    return torch.device("cuda:0")


def bits_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev())


def f16_to_i16(a):
    return np.ascontiguousarray(np.asarray(a, np.float16)).view(np.int16)


def oracle_cache(case):
    """Cache built by the oracle's quantiser (host arrays)."""
    kc, vc, ks, vs = O.alloc_paged_cache(case.num_blocks, case.num_kv_heads, case.head_dim)
    O.quant_append(case.k, case.v, case.slot_mapping, kc, vc, ks, vs)
    return kc, vc, ks, vs


def upload_cache(kc, vc, ks, vs):
    return (torch.from_numpy(kc).to(dev()), torch.from_numpy(vc).to(dev()),
            torch.from_numpy(f16_to_i16(ks)).to(dev()), torch.from_numpy(f16_to_i16(vs)).to(dev()))


def download_cache(t):
    kc, vc, ks, vs = (x.cpu().numpy() for x in t)
    return kc, vc, ks.view(np.float16), vs.view(np.float16)


def gpu_append(case, cache=None, slots=None, k_bits=None, v_bits=None):
    """Run the library's append on the case's K/V (bf16 bits) into `cache`
    (allocated zeroed if None); returns the device cache tuple."""
    if cache is None:
        cache = B.alloc_cache(case.num_blocks, case.num_kv_heads, case.head_dim, dev())
    kb = case.k_bits if k_bits is None else k_bits
    vb = case.v_bits if v_bits is None else v_bits
    sl = case.slot_mapping if slots is None else slots
    k = bits_tensor(kb).view(torch.bfloat16)
    v = bits_tensor(vb).view(torch.bfloat16)
    s = torch.from_numpy(np.ascontiguousarray(sl, np.int32)).to(dev())
    B.kv8_quant_append(k, v, s, *cache)
    return cache


def q_tensor(case, q=None):
    if case.q_dtype == "bf16":
        bits = case.q_bits if q is None else q
        return bits_tensor(bits).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(case.q if q is None else q, np.float32)).to(dev())


def gpu_decode(case, cache, q=None, tokens_per_split=0, block_table=None, context_lens=None,
               max_context_len=None, sm_scale=None, workspace=None, kernel_form=None):
    bt = case.block_table if block_table is None else block_table
    cl = case.context_lens if context_lens is None else context_lens
    mcl = int(np.max(cl)) if max_context_len is None else max_context_len
    qt = q_tensor(case, q)
    b, hq, d = qt.shape
    ws_bytes = B.kv8_decode_workspace_size(b, hq, case.num_kv_heads, d, mcl, tokens_per_split)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev()) if workspace is None else workspace
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=dev())
    B.paged_decode_attn_kv8(qt, *cache,
                            torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to(dev()),
                            torch.from_numpy(np.ascontiguousarray(cl, np.int32)).to(dev()),
                            mcl, out, ws, sm_scale=sm_scale, tokens_per_split=tokens_per_split,
                            kernel_form=form(kernel_form))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_close(out, ref, what=""):
    """Tolerance check in fp32; returns (max_abs, rel_l2)."""
    o = np.asarray(out, np.float32)
    r = np.asarray(ref, np.float64).astype(np.float32)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    diff = o.astype(np.float32) - r
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    print(f"parity margin [{what}]: max|delta| {max_abs:.3e} ({max_abs / MAX_ABS:.3f} of bound), "
          f"rel L2 {rel:.3e} ({rel / REL_L2:.3f} of bound)")
    assert max_abs <= MAX_ABS, f"{what}: max|delta| {max_abs:.3e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    return max_abs, rel


def gpu_prefill(case, cache, q=None, q_start_loc=None, context_lens=None, max_q_len=None,
                block_table=None, max_context_len=None, sm_scale=None):
    """Run paged_prefill_chunk_attn_kv8 on a prefill case (bf16 Q bits
    [Tq, Hq, d]); returns fp32 [Tq, Hq, d] (NaN where the kernel wrote
    nothing)."""
    qsl = case.extra["q_start_loc"] if q_start_loc is None else q_start_loc
    qsl = np.ascontiguousarray(qsl, np.int32)
    bt = case.block_table if block_table is None else block_table
    cl = case.context_lens if context_lens is None else context_lens
    mcl = int(np.max(cl)) if max_context_len is None else max_context_len
    mql = int(np.max(np.diff(qsl))) if max_q_len is None else max_q_len
    qt = bits_tensor(case.q_bits if q is None else q).view(torch.bfloat16)
    tq, hq, d = qt.shape
    out = torch.full((tq, hq, d), float("nan"), dtype=torch.float32, device=dev())
    B.paged_prefill_chunk_attn_kv8(
        qt, torch.from_numpy(qsl).to(dev()), mql, *cache,
        torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to(dev()),
        torch.from_numpy(np.ascontiguousarray(cl, np.int32)).to(dev()),
        mcl, out, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_prefill_rows(case, cache_host, picks, q=None, context_lens=None, gather=None):
    """fp64 oracle output for selected (sequence b, chunk row i) pairs, all
    query heads: the oracle's gather (INT8 unless another code format's
    gather is given), causal rule and softmax applied to those rows only.
    Returns [len(picks), Hq, d]."""
    gather = O.gather_dequant if gather is None else gather
    kc, vc, ks, vs = cache_host
    qv = case.q if q is None else q
    cl = case.context_lens if context_lens is None else context_lens
    qsl = case.extra["q_start_loc"]
    hq, hkv = case.num_q_heads, case.num_kv_heads
    G = hq // hkv
    sm = 1.0 / np.sqrt(case.head_dim)
    res = np.zeros((len(picks), hq, case.head_dim), np.float64)
    for b in sorted({b for b, _ in picks}):
        ctx = int(cl[b])
        lc = int(qsl[b + 1] - qsl[b])
        rows = [(n, i) for n, (bb, i) in enumerate(picks) if bb == b]
        for g in range(hkv):
            k = gather(kc, ks, case.block_table[b], ctx, g)
            v = gather(vc, vs, case.block_table[b], ctx, g)
            for n, i in rows:
                vis = O.causal_visibility(ctx, lc)[i:i + 1]
                for h in range(g * G, g * G + G):
                    qrow = np.asarray(qv[qsl[b] + i, h], np.float64)[None, :]
                    res[n, h] = O.softmax_attention(qrow, k, v, sm, vis)[0]
    return res
