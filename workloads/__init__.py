"""Seeded synthetic inputs for paged grouped-query attention.

This module only draws random tensors and lays them out; it holds none of the
attention arithmetic.  Both the CPU oracle (via the tests) and the HIP path
consume what it produces, so neither side ever supplies inputs to the other.

Shapes follow the workloads the pages measure ("Qwen3-4B / 8B / 32B",
section Architecture Notes: 32 query heads / 8 KV heads / head dim 128 for
Qwen3-4B, 64 query heads with GQA group 8 for Qwen3-32B; 1024-token prompts
with 128-token outputs in the serving-load tables; up to 64 requests in
flight; 4097- and 8192-token long prompts on "Qwen3.5-4B / 9B / 27B").

Pool layout (shared contract of the whole library):
  K pool  [num_blocks, Hkv, D/32, 16, 32]  bf16  (per 32-wide slice of the
          head dimension, 16 token rows of 32 contiguous values)
  V pool  [num_blocks, Hkv, D, 16]  bf16  (transposed: 16 token values per d)
Element d of the K row of the token at in-block offset o sits at
k_cache[block, head, d // 32, o, d % 32].  A token at logical position p of sequence s lives in physical block
block_tables[s, p // 16], at in-block offset p % 16; its slot id is
block * 16 + offset.

Draw order (fixed, generator torch.Generator('cpu') seeded with 42 by
default): lengths -> block permutation -> K pool -> V pool -> Q -> new-token
K/V.  Normals are drawn in fp32, multiplied by sigma and rounded to bf16.  The
K pool is drawn in token-row order [num_blocks, Hkv, 16, D] and then stored in
the sliced layout above, so a given seed fixes the same K row for every token.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK_SIZE = 16
BF16_NAN_BITS = 0x7FC0


@dataclass
class DecodeCase:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    context_lens: torch.Tensor      # int32 [B]; includes the token being decoded
    block_tables: torch.Tensor      # int32 [B, max_blocks]; padding = -1
    k_cache: torch.Tensor           # bf16 [NB, Hkv, D/32, 16, 32]
    v_cache: torch.Tensor           # bf16 [NB, Hkv, D, 16]
    q: torch.Tensor                 # bf16 [B, Hq, D]
    k_new: torch.Tensor             # bf16 [B, Hkv, D]  K of the decoded token
    v_new: torch.Tensor             # bf16 [B, Hkv, D]
    slot_mapping: torch.Tensor      # int64 [B]; slot of position ctx-1
    sigma: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.context_lens.numel())

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode pass must read."""
        return int(self.context_lens.sum()) * 2 * self.num_kv_heads * self.head_dim * 2


@dataclass
class PrefillCase:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    q_lens: list
    prefix_lens_list: list
    cu_seqlens: torch.Tensor        # int32 [S+1] over new tokens
    prefix_lens: torch.Tensor       # int32 [S]
    block_tables: torch.Tensor      # int32 [S, max_blocks]; padding = -1
    k_cache: torch.Tensor           # bf16 [NB, Hkv, D/32, 16, 32]; prefix tokens live
    v_cache: torch.Tensor           # bf16 [NB, Hkv, D, 16]
    q: torch.Tensor                 # bf16 [total_q, Hq, D]
    k_new: torch.Tensor             # bf16 [total_q, Hkv, D]
    v_new: torch.Tensor             # bf16 [total_q, Hkv, D]
    slot_mapping: torch.Tensor      # int64 [total_q]
    sigma: float = 1.0

    @property
    def num_seqs(self) -> int:
        return len(self.q_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def flops(self) -> int:
        """Algorithmic flops: 4*D*Hq per unmasked (query, key) pair."""
        pairs = sum(n * p + n * (n + 1) // 2 for n, p in zip(self.q_lens, self.prefix_lens_list))
        return 4 * self.head_dim * self.num_q_heads * pairs


@dataclass
class MultiDecodeCase:
    """Decode with query_len (T) query tokens per sequence: the pass that
    verifies a block of drafted tokens."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    query_len: int
    context_lens: torch.Tensor      # int32 [B]; includes the T query tokens
    block_tables: torch.Tensor      # int32 [B, max_blocks]; padding = -1
    k_cache: torch.Tensor           # bf16 [NB, Hkv, D/32, 16, 32]
    v_cache: torch.Tensor           # bf16 [NB, Hkv, D, 16]
    q: torch.Tensor                 # bf16 [B, T, Hq, D]
    k_new: torch.Tensor             # bf16 [B*T, Hkv, D]  K of the query tokens
    v_new: torch.Tensor             # bf16 [B*T, Hkv, D]
    slot_mapping: torch.Tensor      # int64 [B*T]; slots of positions ctx-T..ctx-1
    sigma: float = 1.0

    @property
    def batch(self) -> int:
        return int(self.context_lens.numel())

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one pass must read (each cached token once)."""
        return int(self.context_lens.sum()) * 2 * self.num_kv_heads * self.head_dim * 2


def _normal_bf16(g, shape, sigma, device="cpu"):
    if device == "cpu":
        x = torch.randn(*shape, generator=g, dtype=torch.float32)
    else:
        x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    if sigma != 1.0:
        x = x * sigma
    return x.to(torch.bfloat16)


def _k_pool(g, num_blocks, num_kv_heads, head_dim, sigma):
    """K pool drawn as token rows [NB, Hkv, 16, D], stored [NB, Hkv, D/W, 16, W]
    with slice width W = 32 (head dims that are not a multiple of 32, which
    only the oracle's own small cases use, get one slice of width D)."""
    w = 32 if head_dim % 32 == 0 else head_dim
    rows = _normal_bf16(g, (num_blocks, num_kv_heads, BLOCK_SIZE, head_dim), sigma)
    return (rows.view(num_blocks, num_kv_heads, BLOCK_SIZE, head_dim // w, w)
            .permute(0, 1, 3, 2, 4).contiguous())


def _assign_blocks(g, num_blocks, blocks_per_seq, max_blocks, permute=True):
    """Consecutive chunks of a random permutation of the pool, one per sequence."""
    total = sum(blocks_per_seq)
    if total > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {total}")
    perm = torch.randperm(num_blocks, generator=g) if permute else torch.arange(num_blocks)
    bt = torch.full((len(blocks_per_seq), max_blocks), -1, dtype=torch.int32)
    off = 0
    for s, nb in enumerate(blocks_per_seq):
        bt[s, :nb] = perm[off:off + nb].to(torch.int32)
        off += nb
    return bt


def slot_of(block_tables: torch.Tensor, seq: int, pos: int) -> int:
    return int(block_tables[seq, pos // BLOCK_SIZE]) * BLOCK_SIZE + pos % BLOCK_SIZE


def poison_pool(k_cache, v_cache, block_tables, live_lens):
    """Write bf16 NaN into every pool slot that does not hold a live token.

    live_lens[s] = number of positions of sequence s whose K/V must be
    present.  Every other slot (unused blocks, tails of last blocks) becomes
    NaN so that a reader that touches it produces NaN.
    """
    nb = k_cache.shape[0]
    live = torch.zeros(nb, BLOCK_SIZE, dtype=torch.bool)
    for s, n in enumerate(live_lens):
        for p in range(0, int(n), BLOCK_SIZE):
            blk = int(block_tables[s, p // BLOCK_SIZE])
            cnt = min(BLOCK_SIZE, int(n) - p)
            live[blk, :cnt] = True
    dead = ~live
    kv = k_cache.view(torch.int16)
    vv = v_cache.view(torch.int16)
    nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int32).to(torch.int16)
    kv[dead.view(nb, 1, 1, BLOCK_SIZE, 1).expand_as(kv)] = nan  # [NB,Hkv,D/32,16,32]
    vv[dead.unsqueeze(1).unsqueeze(2).expand_as(vv)] = nan    # [NB,Hkv,D,16]


def make_decode_case(name, *, context_lens=None, ctx_range=None, batch=None,
                     num_q_heads, num_kv_heads, head_dim, num_blocks,
                     sigma=1.0, scale=None, seed=42, max_blocks=None,
                     poison=True, permute=True, device="cpu"):
    g = torch.Generator("cpu").manual_seed(seed)
    if context_lens is None:
        lo, hi = ctx_range
        ctx = torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64)
    else:
        ctx = torch.tensor(list(context_lens), dtype=torch.int64)
    nblk = [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    if max_blocks is None:
        max_blocks = max(nblk) if nblk else 1
    bt = _assign_blocks(g, num_blocks, nblk, max_blocks, permute)
    kc = _k_pool(g, num_blocks, num_kv_heads, head_dim, sigma)
    vc = _normal_bf16(g, (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE), sigma)
    B = int(ctx.numel())
    q = _normal_bf16(g, (B, num_q_heads, head_dim), sigma)
    k_new = _normal_bf16(g, (B, num_kv_heads, head_dim), sigma)
    v_new = _normal_bf16(g, (B, num_kv_heads, head_dim), sigma)
    slots = torch.tensor([slot_of(bt, s, int(ctx[s]) - 1) if int(ctx[s]) > 0 else -1
                          for s in range(B)], dtype=torch.int64)
    if poison:
        # The decoded token's own slot is poisoned too: pa_write_kv fills it.
        poison_pool(kc, vc, bt, [int(c) - 1 if int(c) > 0 else 0 for c in ctx])
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeCase(name, num_q_heads, num_kv_heads, head_dim, num_blocks, float(scale),
                      ctx.to(torch.int32), bt, kc, vc, q, k_new, v_new, slots, sigma)


def decode_layer(case: DecodeCase, seed: int, poison=True) -> DecodeCase:
    """Another layer of the same decode step: the same lengths, block table
    and slots, freshly drawn pools, queries and new-token K/V (generator
    seeded with `seed`; draw order K pool -> V pool -> Q -> new-token K/V),
    NaN-poisoned like the original."""
    g = torch.Generator("cpu").manual_seed(seed)
    kc = _k_pool(g, case.num_blocks, case.num_kv_heads, case.head_dim, case.sigma)
    vc = _normal_bf16(g, tuple(case.v_cache.shape), case.sigma)
    q = _normal_bf16(g, tuple(case.q.shape), case.sigma)
    k_new = _normal_bf16(g, tuple(case.k_new.shape), case.sigma)
    v_new = _normal_bf16(g, tuple(case.v_new.shape), case.sigma)
    if poison:
        poison_pool(kc, vc, case.block_tables,
                    [int(c) - 1 if int(c) > 0 else 0 for c in case.context_lens])
    return DecodeCase(f"{case.name}_layer{seed}", case.num_q_heads, case.num_kv_heads,
                      case.head_dim, case.num_blocks, case.scale, case.context_lens.clone(),
                      case.block_tables.clone(), kc, vc, q, k_new, v_new,
                      case.slot_mapping.clone(), case.sigma)


def make_prefill_case(name, *, q_lens, prefix_lens, num_q_heads, num_kv_heads, head_dim,
                      num_blocks, sigma=1.0, scale=None, seed=42, poison=True,
                      permute=True, max_blocks=None):
    g = torch.Generator("cpu").manual_seed(seed)
    q_lens = [int(x) for x in q_lens]
    prefix_lens = [int(x) for x in prefix_lens]
    tot = [n + p for n, p in zip(q_lens, prefix_lens)]
    nblk = [(t + BLOCK_SIZE - 1) // BLOCK_SIZE for t in tot]
    if max_blocks is None:
        max_blocks = max(nblk) if nblk else 1
    bt = _assign_blocks(g, num_blocks, nblk, max_blocks, permute)
    kc = _k_pool(g, num_blocks, num_kv_heads, head_dim, sigma)
    vc = _normal_bf16(g, (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE), sigma)
    total_q = sum(q_lens)
    q = _normal_bf16(g, (total_q, num_q_heads, head_dim), sigma)
    k_new = _normal_bf16(g, (total_q, num_kv_heads, head_dim), sigma)
    v_new = _normal_bf16(g, (total_q, num_kv_heads, head_dim), sigma)
    slots = []
    for s, (n, p) in enumerate(zip(q_lens, prefix_lens)):
        slots += [slot_of(bt, s, p + i) for i in range(n)]
    slots = torch.tensor(slots, dtype=torch.int64)
    cu = torch.zeros(len(q_lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(q_lens, dtype=torch.int32), 0)
    if poison:
        poison_pool(kc, vc, bt, prefix_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PrefillCase(name, num_q_heads, num_kv_heads, head_dim, num_blocks, float(scale),
                       q_lens, prefix_lens, cu, torch.tensor(prefix_lens, dtype=torch.int32),
                       bt, kc, vc, q, k_new, v_new, slots, sigma)


def make_multi_decode_case(name, *, query_len, context_lens=None, ctx_range=None, batch=None,
                           num_q_heads, num_kv_heads, head_dim, num_blocks, sigma=1.0,
                           scale=None, seed=42, max_blocks=None, poison=True, permute=True):
    """Same draw order as make_decode_case; q is [B, T, Hq, D] and the T
    query tokens' K/V (positions ctx-T..ctx-1) are drawn as k_new/v_new.
    A sequence with 0 < ctx < T (invalid) gets slot -1 for positions < 0."""
    g = torch.Generator("cpu").manual_seed(seed)
    T = int(query_len)
    if context_lens is None:
        lo, hi = ctx_range
        ctx = torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64)
    else:
        ctx = torch.tensor(list(context_lens), dtype=torch.int64)
    nblk = [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    if max_blocks is None:
        max_blocks = max(nblk) if nblk else 1
    bt = _assign_blocks(g, num_blocks, nblk, max_blocks, permute)
    kc = _k_pool(g, num_blocks, num_kv_heads, head_dim, sigma)
    vc = _normal_bf16(g, (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE), sigma)
    B = int(ctx.numel())
    q = _normal_bf16(g, (B, T, num_q_heads, head_dim), sigma)
    k_new = _normal_bf16(g, (B * T, num_kv_heads, head_dim), sigma)
    v_new = _normal_bf16(g, (B * T, num_kv_heads, head_dim), sigma)
    slots = []
    for s in range(B):
        n = int(ctx[s])
        slots += [slot_of(bt, s, n - T + t) if n - T + t >= 0 else -1 for t in range(T)]
    slots = torch.tensor(slots, dtype=torch.int64)
    if poison:
        poison_pool(kc, vc, bt, [max(int(c) - T, 0) for c in ctx])
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return MultiDecodeCase(name, num_q_heads, num_kv_heads, head_dim, num_blocks, float(scale),
                           T, ctx.to(torch.int32), bt, kc, vc, q, k_new, v_new, slots, sigma)


# ---------------------------------------------------------------------------
# The five workloads.  Sizes are the ones the serving pages measure on, per
# the shapes listed in the module docstring.
# ---------------------------------------------------------------------------

def tiny_decode(seed=42, poison=True):
    """2 sequences (context 37 and 50), 4/2 heads, head_dim 64, 16-block pool."""
    return make_decode_case("tiny_decode", context_lens=[37, 50], num_q_heads=4,
                            num_kv_heads=2, head_dim=64, num_blocks=16, max_blocks=4,
                            scale=1.0 / 8.0, seed=seed, poison=poison)


def qwen3_4b_decode(seed=42, poison=True):
    """Batch 8, context U{1024..1152}, 32/8 heads, head_dim 128, 4096-block pool."""
    return make_decode_case("qwen3_4b_decode_b8", ctx_range=(1024, 1152), batch=8,
                            num_q_heads=32, num_kv_heads=8, head_dim=128, num_blocks=4096,
                            max_blocks=72, seed=seed, poison=poison)


def qwen3_4b_prefill(seed=42, poison=True):
    """4 x 1024 new tokens, sequences 1 and 3 hit a 512-token cached prefix."""
    return make_prefill_case("qwen3_4b_prefill_4x1024", q_lens=[1024] * 4,
                             prefix_lens=[0, 512, 0, 512], num_q_heads=32, num_kv_heads=8,
                             head_dim=128, num_blocks=4096, seed=seed, poison=poison)


def qwen3_32b_decode(seed=42, poison=True):
    """Batch 64, context U{1024..1152}, 64/8 heads (group 8), head_dim 128."""
    return make_decode_case("qwen3_32b_decode_b64", ctx_range=(1024, 1152), batch=64,
                            num_q_heads=64, num_kv_heads=8, head_dim=128, num_blocks=8192,
                            max_blocks=72, seed=seed, poison=poison)


def qwen3_32b_decode_long(seed=42, poison=True):
    """Batch 4 at 8192 tokens: the split-K case."""
    return make_decode_case("qwen3_32b_decode_b4_8192", context_lens=[8192] * 4,
                            num_q_heads=64, num_kv_heads=8, head_dim=128, num_blocks=8192,
                            seed=seed, poison=poison)


def qwen3_32b_decode_mixed(seed=42, poison=True):
    """One 8192-token request decoding among seven ordinary ones (contexts
    U{1024..1152}), Qwen3-32B heads: a batch of mixed lengths as continuous
    batching produces it (the long-prompt lengths of "Qwen3.5-4B / 9B /
    27B" beside the 1024-token serving prompts)."""
    g = torch.Generator("cpu").manual_seed(seed)
    lens = [8192] + torch.randint(1024, 1153, (7,), generator=g).tolist()
    return make_decode_case("qwen3_32b_decode_mixed_b8", context_lens=lens, num_q_heads=64,
                            num_kv_heads=8, head_dim=128, num_blocks=2048, seed=seed,
                            poison=poison)


def hybrid_decode(seed=42, poison=True):
    """Full-attention layer of a hybrid model: 16/2 heads, head_dim 256, sigma 0.5,
    batch 8 with contexts 4097 and 8192 interleaved."""
    return make_decode_case("hybrid_decode_b8", context_lens=[4097, 8192] * 4,
                            num_q_heads=16, num_kv_heads=2, head_dim=256, num_blocks=8192,
                            sigma=0.5, scale=1.0 / 16.0, seed=seed, poison=poison)


def hybrid_prefill(seed=42, poison=True):
    """One 4097-token causal prefill, no prefix, 16/2 heads, head_dim 256, sigma 0.5."""
    return make_prefill_case("hybrid_prefill_4097", q_lens=[4097], prefix_lens=[0],
                             num_q_heads=16, num_kv_heads=2, head_dim=256, num_blocks=8192,
                             sigma=0.5, scale=1.0 / 16.0, seed=seed, poison=poison)


def qwen3_4b_verify(batch=4, seed=42, poison=True):
    """Verifying a drafted block on Qwen3-4B: the last accepted token plus 7
    drafted ones (T = 8) per sequence, batch 4 (the pages' concurrency 4; 1
    for single-stream), context U{1024..1152}, 32/8 heads, head_dim 128."""
    return make_multi_decode_case(f"qwen3_4b_verify_b{batch}_t8", query_len=8,
                                  ctx_range=(1024, 1152), batch=batch, num_q_heads=32,
                                  num_kv_heads=8, head_dim=128, num_blocks=4096, max_blocks=72,
                                  seed=seed, poison=poison)


DECODE_CASES = {
    "tiny_decode": tiny_decode,
    "qwen3_4b_decode_b8": qwen3_4b_decode,
    "qwen3_32b_decode_b64": qwen3_32b_decode,
    "qwen3_32b_decode_b4_8192": qwen3_32b_decode_long,
    "hybrid_decode_b8": hybrid_decode,
}

PREFILL_CASES = {
    "qwen3_4b_prefill_4x1024": qwen3_4b_prefill,
    "hybrid_prefill_4097": hybrid_prefill,
}
