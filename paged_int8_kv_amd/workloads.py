"""Seeded synthetic inputs for the paged INT8-KV attention path.

This module only draws random numbers and lays them out (sequence lengths,
bf16 K/V/Q values, block tables, slot mappings).  It holds none of the
method's arithmetic: no quantisation, no attention.  Both the HIP path and
the CPU oracle receive their inputs from here, and neither side imports the
other.

Shapes follow the pages' models: Llama-3.1-8B attention is 32 query heads
over 8 KV heads of dimension 128, Llama-3-70B is 64 over 8 (the GQA model
table of "KV Cache 优化全景解析" section 3.3).  Blocks hold 16 tokens
(section 6.3 of the same page).  Key outlier channels mimic the per-channel
outliers that the same page describes for the key cache in section 7.1.

Draw order for a case (numpy PCG64 seeded with the config's seed):
context lengths, key outlier channels, Q, K, V, then the physical block
permutation.  Values are drawn as fp32 N(0, 1), scaled by 10 on outlier
channels where asked, and rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16


def to_bf16(x):
    """Round fp32 values to bf16 (nearest even).  Returns (values as fp32,
    raw uint16 bit patterns)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.to(torch.float32).numpy(), bits


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32 values."""
    bits = np.asarray(bits, np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class PagedCase:
    """One synthetic batch for the paged cache.

    Token order in k/v/slot_mapping is sequence-major: all tokens of
    sequence 0 (positions 0..ctx0-1), then sequence 1, and so on.
    """
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str                 # "f32" or "bf16"
    context_lens: np.ndarray     # int32 [B]
    block_table: np.ndarray      # int32 [B, max_blocks]
    num_blocks: int
    q: np.ndarray                # fp32 values [B or Tq, Hq, d]
    q_bits: np.ndarray | None    # uint16 bf16 bits when q_dtype == "bf16"
    k: np.ndarray                # fp32 (bf16-exact) [Ntok, Hkv, d]
    v: np.ndarray
    k_bits: np.ndarray           # uint16 [Ntok, Hkv, d]
    v_bits: np.ndarray
    slot_mapping: np.ndarray     # int32 [Ntok]
    token_seq: np.ndarray        # int32 [Ntok] sequence of each token
    token_pos: np.ndarray        # int32 [Ntok] position inside its sequence
    outlier_channels: np.ndarray | None = None   # int [Hkv, 4] for K
    extra: dict = field(default_factory=dict)

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self):
        return self.block_table.shape[1]


def _slots_for(block_table, seq_ids, positions):
    return (block_table[seq_ids, positions // BLOCK_SIZE] * BLOCK_SIZE
            + positions % BLOCK_SIZE).astype(np.int32)


def make_paged_case(*, batch, num_q_heads, num_kv_heads, head_dim, context_lens,
                    q_dtype="bf16", q_rows=None, k_outliers=False,
                    outlier_factor=10.0, seed=0, permute=True,
                    headroom_tokens=0, spare_blocks=0):
    """Build a case.  context_lens: int array [B] or a callable rng -> [B]
    (drawn first).  q_rows: rows of Q (default: one per sequence, decode).
    headroom_tokens: extra table capacity per sequence for later appends.
    spare_blocks: unused physical blocks mixed into the pool."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if callable(context_lens):
        ctx = np.asarray(context_lens(rng), np.int64)
    else:
        ctx = np.asarray(context_lens, np.int64)
    assert ctx.shape == (batch,)
    d = head_dim
    outl = None
    if k_outliers:
        outl = np.stack([rng.choice(d, size=4, replace=False)
                         for _ in range(num_kv_heads)])
    nq = batch if q_rows is None else q_rows
    q = rng.standard_normal((nq, num_q_heads, d), dtype=np.float32)
    ntok = int(ctx.sum())
    k = rng.standard_normal((ntok, num_kv_heads, d), dtype=np.float32)
    v = rng.standard_normal((ntok, num_kv_heads, d), dtype=np.float32)
    if outl is not None:
        for h in range(num_kv_heads):
            k[:, h, outl[h]] *= np.float32(outlier_factor)
    blocks_per_seq = -(-(ctx + headroom_tokens) // BLOCK_SIZE)
    max_blocks = max(1, int(blocks_per_seq.max()))
    nb = int(blocks_per_seq.sum()) + spare_blocks
    phys = rng.permutation(nb) if permute else np.arange(nb)
    table = np.zeros((batch, max_blocks), np.int32)
    cur = 0
    for b in range(batch):
        n = int(blocks_per_seq[b])
        table[b, :n] = phys[cur:cur + n]
        cur += n
    seq = np.repeat(np.arange(batch), ctx).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]])
    pos = (np.arange(ntok) - np.repeat(starts, ctx)).astype(np.int32)
    slots = _slots_for(table, seq, pos)
    kv, kb = to_bf16(k)
    vv, vb = to_bf16(v)
    if q_dtype == "bf16":
        qv, qb = to_bf16(q)
    else:
        qv, qb = q, None
    return PagedCase(batch, num_q_heads, num_kv_heads, d, q_dtype,
                     ctx.astype(np.int32), table, nb, qv, qb, kv, vv, kb, vb,
                     slots, seq, pos, outl)


def paged_bf16_cache(case, poison_unused=False):
    """The case's bf16 K/V tokens laid out as a paged 16-bit cache: bit
    patterns [NB, Hkv, 16, d] (uint16) for K and V, token n in the slot
    slot_mapping[n] names.  Slots that no token uses hold 0, or a NaN
    pattern when poison_unused."""
    shape = (case.num_blocks, case.num_kv_heads, BLOCK_SIZE, case.head_dim)
    fill = np.uint16(0x7FC1) if poison_unused else np.uint16(0)
    kc = np.full(shape, fill, np.uint16)
    vc = np.full(shape, fill, np.uint16)
    blk, off = case.slot_mapping // BLOCK_SIZE, case.slot_mapping % BLOCK_SIZE
    kc[blk, :, off, :] = case.k_bits
    vc[blk, :, off, :] = case.v_bits
    return kc, vc


# ---------------------------------------------------------------------------
# The five workloads of this path
# ---------------------------------------------------------------------------
def tiny_decode(seed=1):
    """Batch 1, 4 query heads over 1 KV head, d=64, 256 tokens, identity
    block table, fp32 Q."""
    return make_paged_case(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                           context_lens=[256], q_dtype="f32", seed=seed,
                           permute=False)


def llama8b_decode(seed=2, batch=32, lo=1024, hi=4096):
    """Llama-3.1-8B-shaped decode layer: batch 32, 32/8 heads, d=128,
    context lengths uniform integers in [1024, 4096], bf16 Q, four K outlier
    channels per KV head scaled by 10, permuted physical blocks."""
    return make_paged_case(batch=batch, num_q_heads=32, num_kv_heads=8,
                           head_dim=128,
                           context_lens=lambda r: r.integers(lo, hi + 1, size=batch),
                           q_dtype="bf16", k_outliers=True, seed=seed)


def long_context_decode(seed=3, batch=4, ctx=32768, steps=64):
    """Long-context decode with append: batch 4, 32/8 heads, d=128, 32768
    tokens each, table headroom for `steps` appended tokens per sequence,
    fp32 Q, K/V N(0,1).  extra['step_k'/'step_v'] hold the appended tokens
    as bf16 [steps, B, Hkv, d], extra['step_q'] the per-step queries."""
    case = make_paged_case(batch=batch, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, context_lens=[ctx] * batch,
                           q_dtype="f32", seed=seed, headroom_tokens=steps)
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    sk = rng.standard_normal((steps, batch, 8, 128), dtype=np.float32)
    sv = rng.standard_normal((steps, batch, 8, 128), dtype=np.float32)
    sq = rng.standard_normal((steps, batch, 32, 128), dtype=np.float32)
    case.extra["step_k"], case.extra["step_k_bits"] = to_bf16(sk)
    case.extra["step_v"], case.extra["step_v_bits"] = to_bf16(sv)
    case.extra["step_q"] = sq
    case.extra["steps"] = steps
    return case


def step_slots(case, step):
    """Slots of the token appended at `step` (0-based) of a long-context
    case: position context_lens[b] + step of each sequence."""
    pos = case.context_lens.astype(np.int64) + step
    b = np.arange(case.batch)
    return _slots_for(case.block_table, b, pos)


def llama70b_layer_lens(layer, batch=64, lo=512, hi=16384, seed=4):
    """Context lengths of one layer of the Llama-3-70B sweep:
    floor(exp(U(ln 512, ln 16384)))."""
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + layer))
    return np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi), size=batch))).astype(np.int32)


def llama70b_layer(layer, seed=4, batch=64):
    """One layer of the Llama-3-70B sweep on the host (tests at reduced
    batch use this): 64/8 heads, d=128, log-uniform lengths, K outliers,
    bf16 Q, independent permuted table per layer."""
    lens = llama70b_layer_lens(layer, batch=batch, seed=seed)
    return make_paged_case(batch=batch, num_q_heads=64, num_kv_heads=8,
                           head_dim=128, context_lens=lens, q_dtype="bf16",
                           k_outliers=True, seed=seed * 100000 + layer)


def chunked_prefill(seed=5, batch=8, chunk=512, lo=2048, hi=8192,
                    num_q_heads=32, num_kv_heads=8, head_dim=128):
    """Chunked prefill: existing context of uniform integer length in
    [2048, 8192] per sequence, then a causal chunk of 512 query rows whose
    own K/V are appended first.  K/V of context and chunk are drawn together
    (sequence-major, chunk tokens last in each sequence); bf16 Q/K/V N(0,1).
    extra['q_start_loc'] [B+1], extra['ctx_prev'] [B], extra['chunk_mask']
    marks the chunk tokens inside k/v/slot_mapping."""
    rng = np.random.Generator(np.random.PCG64(seed))
    prev = rng.integers(lo, hi + 1, size=batch)
    case = make_paged_case(batch=batch, num_q_heads=num_q_heads,
                           num_kv_heads=num_kv_heads, head_dim=head_dim,
                           context_lens=prev + chunk, q_dtype="bf16",
                           q_rows=batch * chunk, seed=seed + 1)
    case.extra["ctx_prev"] = prev.astype(np.int32)
    case.extra["q_start_loc"] = (np.arange(batch + 1) * chunk).astype(np.int32)
    case.extra["chunk_mask"] = case.token_pos >= np.repeat(prev, prev + chunk)
    case.extra["chunk"] = chunk
    return case


def prefill_case(ctx_prev, chunk_lens, *, num_q_heads=32, num_kv_heads=8, head_dim=128,
                 seed=6, k_outliers=False, spare_blocks=0, permute=True):
    """Ragged chunked prefill: sequence b holds ctx_prev[b] earlier tokens
    and a chunk of chunk_lens[b] rows (0 allowed) whose K/V are in the cache
    too, so context_lens = ctx_prev + chunk_lens.  Q rows of all chunks are
    packed in sequence order; extra['q_start_loc'] [B+1], extra['max_q_len'].
    bf16 Q/K/V N(0,1)."""
    prev = np.asarray(ctx_prev, np.int64)
    lens = np.asarray(chunk_lens, np.int64)
    batch = len(prev)
    case = make_paged_case(batch=batch, num_q_heads=num_q_heads,
                           num_kv_heads=num_kv_heads, head_dim=head_dim,
                           context_lens=prev + lens, q_dtype="bf16",
                           q_rows=max(1, int(lens.sum())), seed=seed,
                           k_outliers=k_outliers, spare_blocks=spare_blocks,
                           permute=permute)
    case.extra["ctx_prev"] = prev.astype(np.int32)
    case.extra["q_start_loc"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    case.extra["max_q_len"] = int(lens.max()) if batch else 0
    return case


def llama70b_layer_device(layer, device, batch=64, seed=4):
    """One layer of the Llama-3-70B sweep with its K/V/Q drawn on the device
    (the full sweep holds tens of GB of cache).  Context lengths, key outlier
    channels and the permuted block table come from numpy (PCG64 seeded
    seed * 100000 + layer, drawn in that order); K, V and Q are drawn fp32
    N(0, 1) on the device by torch.Generator seeded 4000 + layer (K, then V,
    then Q), outlier channels of K scaled by 10, rounded to bf16.
    Returns a dict: context_lens, block_table, num_blocks (numpy),
    outlier_channels, token_seq, token_pos, slot_mapping (numpy int32), and
    device tensors k, v [Ntok, 8, 128] and q [B, 64, 128] (bf16)."""
    import torch
    lens = llama70b_layer_lens(layer, batch=batch, seed=seed).astype(np.int64)
    rng = np.random.Generator(np.random.PCG64(seed * 100000 + layer))
    hkv, d = 8, 128
    outl = np.stack([rng.choice(d, size=4, replace=False) for _ in range(hkv)])
    blocks_per_seq = -(-lens // BLOCK_SIZE)
    nb = int(blocks_per_seq.sum())
    phys = rng.permutation(nb)
    table = np.zeros((batch, int(blocks_per_seq.max())), np.int32)
    cur = 0
    for b in range(batch):
        n = int(blocks_per_seq[b])
        table[b, :n] = phys[cur:cur + n]
        cur += n
    seq = np.repeat(np.arange(batch), lens).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    pos = (np.arange(int(lens.sum())) - np.repeat(starts, lens)).astype(np.int32)
    slots = _slots_for(table, seq, pos)
    g = torch.Generator(device=device)
    g.manual_seed(4000 + layer)
    ntok = int(lens.sum())
    k = torch.randn((ntok, hkv, d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((ntok, hkv, d), generator=g, device=device, dtype=torch.float32)
    q = torch.randn((batch, 64, d), generator=g, device=device, dtype=torch.float32)
    for h in range(hkv):
        idx = torch.from_numpy(outl[h]).to(device)
        k[:, h, idx] *= 10.0
    return dict(context_lens=lens.astype(np.int32), block_table=table, num_blocks=nb,
                outlier_channels=outl, token_seq=seq, token_pos=pos, slot_mapping=slots,
                k=k.to(torch.bfloat16), v=v.to(torch.bfloat16), q=q.to(torch.bfloat16))


def long_context_258k(batch, device, ctx=258 * 1024, seed=7, num_q_heads=32, num_kv_heads=8,
                      head_dim=128):
    """Sequences of 258K tokens each for the equal-memory-budget comparison
    ("KV-Cache 全栈优化系统" README, section 实验效果（摘要）: 258K context,
    same GPU-memory budget), Llama-3.1-8B attention shape.  The block table
    (a PCG64(seed) permutation of all blocks) and the key outlier channels
    come from numpy; the tokens of sequence b are drawn on the device by
    torch.Generator seeded seed * 1000 + b (K, then V; fp32 N(0, 1), the 4
    outlier channels of each KV head of K scaled by 10, rounded to bf16), so
    sequence b holds the same tokens whatever the batch.  Q row b [Hq, d] is
    drawn N(0, 1) by a generator seeded seed * 1000 + 500 + b, rounded to bf16.
    Returns a dict: context_lens, block_table, num_blocks, outlier_channels
    (numpy), q (device bf16), tokens(b) -> (k, v) device bf16 [ctx, Hkv, d],
    and slots(b) -> device int32 [ctx] physical slots of sequence b."""
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    d, hkv = head_dim, num_kv_heads
    outl = np.stack([rng.choice(d, size=4, replace=False) for _ in range(hkv)])
    nbs = -(-ctx // BLOCK_SIZE)
    nb = batch * nbs
    table = rng.permutation(nb).astype(np.int32).reshape(batch, nbs)
    lens = np.full(batch, ctx, np.int32)
    qs = []
    for b in range(batch):
        gq = torch.Generator(device=device)
        gq.manual_seed(seed * 1000 + 500 + b)
        qs.append(torch.randn((num_q_heads, d), generator=gq, device=device,
                              dtype=torch.float32))
    q = torch.stack(qs).to(torch.bfloat16)
    outl_t = [torch.from_numpy(outl[h]).to(device) for h in range(hkv)]
    table_t = torch.from_numpy(table).to(device)

    def tokens(b):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1000 + b)
        k = torch.randn((ctx, hkv, d), generator=g, device=device, dtype=torch.float32)
        v = torch.randn((ctx, hkv, d), generator=g, device=device, dtype=torch.float32)
        for h in range(hkv):
            k[:, h, outl_t[h]] *= 10.0
        return k.to(torch.bfloat16), v.to(torch.bfloat16)

    def slots(b):
        pos = torch.arange(ctx, device=device, dtype=torch.int64)
        return (table_t[b].long()[pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE).to(torch.int32)

    return dict(context_lens=lens, block_table=table, num_blocks=nb, outlier_channels=outl,
                q=q, tokens=tokens, slots=slots)


def rope_cos_sin(max_position, head_dim, base=500000.0):
    """The rotary-embedding table a serving engine keeps: fp32 [max_position,
    head_dim], row p = cos(p * theta_j) for j < d/2, then sin(p * theta_j),
    theta_j = base^(-2j/d) (Llama-3's base 500000), computed in fp64 and
    rounded to fp32."""
    inv = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
