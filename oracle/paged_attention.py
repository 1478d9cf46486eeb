"""CPU fp64 oracle for grouped-query attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code,
constants or helpers with the HIP library; the only thing both sides use is
the seeded input generator in workloads/, which holds no attention
arithmetic.

What is computed (the pages print no formula; this is the plainest reading):
  * "Qwen3-4B / 8B / 32B", section Architecture Notes: full attention with
    grouped-query attention -- Hq query heads share Hkv key/value heads
    (32/8 for Qwen3-4B, group 8 for Qwen3-32B).  Query head h reads KV head
    h // (Hq / Hkv) (consecutive groups).
  * Same page, intro and Architecture Notes: the KV cache is paged.  Blocks
    hold 16 tokens; a per-sequence block table maps logical block p // 16 to a
    physical block of the pool.
  * Same page, section Warm Prefix-Cache TTFT and Architecture Notes (prefix
    cache on by default): a prefill whose prompt starts with cached blocks
    computes only the new tokens, which attend to the cached prefix and,
    causally, to each other.
  * Same page, section DSpark Speculative Decoding: the target model checks
    a block of drafted tokens in one pass.  Read here as decode with T query
    tokens per sequence, all already appended to the cache: token t of T
    sits at position ctx - T + t and sees keys 0..ctx - T + t (causal within
    the block, full over the cached context), exactly as those tokens would
    be computed as a prefill whose cached prefix is the first ctx - T tokens.
  * Same page, section KV Offload: sealed KV blocks are restored from a
    host tier instead of recomputing the prefill.  Read as a block-granular
    copy: destination block d_i of a pool (or of a packed buffer of blocks)
    receives source block s_i, K and V of every KV head, bit for bit; a copy
    that names a block outside either side is skipped.  The same copy makes a
    private duplicate of a shared prefix block inside one pool.
  * Attention itself is scaled dot-product softmax attention:
      z_j = scale * <q, k_j>,   w_j = exp(z_j) / sum_i exp(z_i),
      out = sum_j w_j v_j,
    evaluated here in fp64 with the maximum subtracted before exp (which
    changes nothing mathematically).

Layout contract (also defined by the library header):
  K pool [NB, Hkv, D/W, 16, W] with slice width W = 32 in the library: K of
      the token in (block b, offset o) for KV head g is k_cache[b, g, :, o, :]
      read slice by slice, element d at k_cache[b, g, d // W, o, d % W].  W
      is taken from the pool's last axis, so tiny cases whose D is not a
      multiple of 32 use a single slice of width D.
  V pool [NB, Hkv, D, 16]: V of that token is v_cache[b, g, :, o].
  slot id = b * 16 + o; a negative slot means "do not write".

Every input that carries bf16 data is passed as uint16 bit patterns; the
oracle widens them to fp64 exactly.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(brute force in 50-digit arithmetic on tiny inputs, closed forms, invariants
and hand-derived golden cases).
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


# ---------------------------------------------------------------------------
# bf16 <-> fp64
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp64."""
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_f64(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64.

    bf16 keeps 8 significant bits: with x = m * 2**e, 0.5 <= |m| < 1, the
    representable neighbours are multiples of 2**(e-8).  np.rint rounds half
    to even.  Normal range only (the attention outputs here never approach
    the bf16 subnormal range).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (2**(e-8) for |x| in [2**(e-1), 2**e))."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x == 0, np.finfo(np.float64).tiny, x))
    return np.ldexp(1.0, e - 8)


# ---------------------------------------------------------------------------
# Pieces of the definition (kept small and named, so each can be read
# against the text above)
# ---------------------------------------------------------------------------

def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: consecutive groups of Hq/Hkv query heads."""
    return h // (num_q_heads // num_kv_heads)


def token_location(block_table_row, pos: int):
    """(physical block, in-block offset) of logical position pos."""
    return int(block_table_row[pos // BLOCK]), pos % BLOCK


def read_k(k_cache, block: int, off: int):
    """K rows of all KV heads of one token: [Hkv, D] (the D/W slices in
    order)."""
    hkv = k_cache.shape[1]
    return k_cache[block, :, :, off, :].reshape(hkv, -1)


def read_v(v_cache, block: int, off: int):
    """V rows of all KV heads of one token: [Hkv, D]."""
    return v_cache[block, :, :, off]


def slot_location(slot: int):
    """(physical block, in-block offset) named by a slot id."""
    return slot // BLOCK, slot % BLOCK


def scores(q_rows_h: np.ndarray, K_g: np.ndarray, scale: float) -> np.ndarray:
    """z[r, j] = scale * <q_r, k_j> for one query head and its KV head."""
    return scale * (q_rows_h @ K_g.T)


def causal_visible(prefix_len: int, n_new: int) -> np.ndarray:
    """Keys visible to each new token: new token i (absolute position
    prefix_len + i) sees positions 0..prefix_len+i, its own included."""
    return prefix_len + np.arange(n_new) + 1


def gather_sequence(k_cache, v_cache, block_table_row, n: int):
    """K, V of logical positions 0..n-1 of one sequence, as fp64 [n, Hkv, D].

    Only the n live positions are touched; nothing else in the pool (unused
    blocks, tails, table padding) is read.
    """
    hkv, d = k_cache.shape[1], k_cache.shape[2] * k_cache.shape[4]
    K = np.empty((n, hkv, d), dtype=np.float64)
    V = np.empty((n, hkv, d), dtype=np.float64)
    for p in range(n):
        b, o = token_location(block_table_row, p)
        K[p] = bf16_bits_to_f64(read_k(k_cache, b, o))
        V[p] = bf16_bits_to_f64(read_v(v_cache, b, o))
    return K, V


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """exp(z - max) / sum over the last axis; rows that are all -inf give 0."""
    m = np.max(z, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m)
    s = np.sum(e, axis=-1, keepdims=True)
    return np.divide(e, s, out=np.zeros_like(e), where=s > 0)


def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           visible: np.ndarray, num_q_heads: int, num_kv_heads: int,
           row_chunk: int = 512) -> np.ndarray:
    """Softmax attention of n query rows over one sequence's keys.

    q_rows [n, Hq, D] fp64; K, V [L, Hkv, D] fp64; visible[r] = number of
    leading keys row r may see (keys j < visible[r]).  Returns [n, Hq, D].
    Rows are processed in chunks only to bound memory.
    """
    n = q_rows.shape[0]
    L = K.shape[0]
    out = np.zeros(q_rows.shape, dtype=np.float64)
    j = np.arange(L)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        mask = j[None, :] < np.asarray(visible[r0:r1])[:, None]      # [r, L]
        for h in range(num_q_heads):
            g = kv_head_of(h, num_q_heads, num_kv_heads)
            z = scores(q_rows[r0:r1, h, :], K[:, g, :], scale)        # [r, L]
            z = np.where(mask, z, -np.inf)
            w = softmax_rows(z)
            out[r0:r1, h, :] = w @ V[:, g, :]
    return out


# ---------------------------------------------------------------------------
# The four operations of the library
# ---------------------------------------------------------------------------

def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping):
    """Slot-mapped KV append: returns new pools with token t's K/V written to
    slot slot_mapping[t] (skipped when negative).  Pure bit copies."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        b, o = slot_location(slot)
        kc[b, :, :, o, :] = np.asarray(k_new[t]).reshape(kc.shape[1], kc.shape[2], kc.shape[4])
        vc[b, :, :, o] = v_new[t]
    return kc, vc


def decode(q, k_cache, v_cache, block_tables, context_lens, scale,
           num_q_heads, num_kv_heads) -> np.ndarray:
    """One query token per sequence at position ctx-1, attending to keys
    0..ctx-1 (itself included).  q: bf16 bits [B, Hq, D].  Returns fp64."""
    qf = bf16_bits_to_f64(q)
    B = qf.shape[0]
    out = np.zeros(qf.shape, dtype=np.float64)
    for s in range(B):
        n = int(context_lens[s])
        if n <= 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], n)
        out[s] = attend(qf[s:s + 1], K, V, scale, np.array([n]),
                        num_q_heads, num_kv_heads)[0]
    return out


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale,
                    num_q_heads, num_kv_heads, partition_size, num_partitions):
    """Split-K pieces of decode.  Partition p of sequence s covers positions
    [p*ps, (p+1)*ps) clipped to [0, ctx).  For each (s, h, p):
        part_out = sum_{j in p} exp(z_j) v_j / sum_{j in p} exp(z_j)
        part_lse = log sum_{j in p} exp(z_j)          (natural log)
    An empty partition gives part_out = 0 and part_lse = -inf."""
    qf = bf16_bits_to_f64(q)
    B, Hq, D = qf.shape
    P = num_partitions
    part_out = np.zeros((B, Hq, P, D), dtype=np.float64)
    part_lse = np.full((B, Hq, P), -np.inf, dtype=np.float64)
    for s in range(B):
        n = int(context_lens[s])
        if n <= 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], n)
        for p in range(P):
            lo, hi = p * partition_size, min(n, (p + 1) * partition_size)
            if lo >= hi:
                continue
            for h in range(Hq):
                g = kv_head_of(h, Hq, num_kv_heads)
                z = scores(qf[s, h, :][None, :], K[lo:hi, g, :], scale)[0]
                m = np.max(z)
                e = np.exp(z - m)
                part_out[s, h, p] = (e @ V[lo:hi, g, :]) / np.sum(e)
                part_lse[s, h, p] = m + np.log(np.sum(e))
    return part_out, part_lse


def combine_partials(part_out, part_lse) -> np.ndarray:
    """Log-sum-exp combination of split-K pieces:
        out = sum_p exp(lse_p) O_p / sum_p exp(lse_p)
    (max-shifted); all partitions empty gives 0.  part_out [..., P, D],
    part_lse [..., P] (any leading dimensions: [B, Hq] or [B, T, Hq])."""
    lse = np.asarray(part_lse, dtype=np.float64)
    po = np.asarray(part_out, dtype=np.float64)
    M = np.max(lse, axis=-1, keepdims=True)
    M = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lse - M)                                    # [..., P]
    den = np.sum(w, axis=-1)
    num = np.einsum("...p,...pd->...d", w, po)
    return np.divide(num, den[..., None], out=np.zeros_like(num), where=den[..., None] > 0)


def prefill(q, k_cache, v_cache, block_tables, cu_seqlens, prefix_lens, scale,
            num_q_heads, num_kv_heads) -> np.ndarray:
    """Varlen causal prefill over paged K/V with cached prefixes.

    Sequence s has N_s = cu[s+1]-cu[s] new tokens after P_s cached ones; its
    new tokens' K/V are already in the pool.  New token i sits at absolute
    position P_s + i and sees keys 0..P_s+i.  q: bf16 bits [total_q, Hq, D].
    Returns fp64 [total_q, Hq, D]."""
    qf = bf16_bits_to_f64(q)
    out = np.zeros(qf.shape, dtype=np.float64)
    S = len(prefix_lens)
    for s in range(S):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        N, P = b - a, int(prefix_lens[s])
        if N <= 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], P + N)
        visible = causal_visible(P, N)
        out[a:b] = attend(qf[a:b], K, V, scale, visible, num_q_heads, num_kv_heads)
    return out


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, scale,
                 num_q_heads, num_kv_heads) -> np.ndarray:
    """Decode with T query tokens per sequence (verifying a drafted block).

    q: bf16 bits [B, T, Hq, D].  context_lens[s] counts all cached tokens of
    sequence s, its T query tokens included.  Token t sits at position
    ctx - T + t and sees keys 0..ctx - T + t.  ctx == 0 gives zeros;
    0 < ctx < T (query tokens at negative positions) gives NaN.
    Returns fp64 [B, T, Hq, D]."""
    qf = bf16_bits_to_f64(q)
    B, T = qf.shape[0], qf.shape[1]
    out = np.zeros(qf.shape, dtype=np.float64)
    for s in range(B):
        n = int(context_lens[s])
        if n == 0:
            continue
        if n < T:
            out[s] = np.nan
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], n)
        visible = causal_visible(n - T, T)
        out[s] = attend(qf[s], K, V, scale, visible, num_q_heads, num_kv_heads)
    return out


def decode_multi_partials(q, k_cache, v_cache, block_tables, context_lens, scale,
                          num_q_heads, num_kv_heads, partition_size, num_partitions):
    """Split-K pieces of decode_multi.  For token t of sequence s the visible
    keys are [0, ctx - T + t + 1); partition p covers [p*ps, (p+1)*ps) of
    them.  For each (s, t, h, p):
        part_out = sum_{j in p, visible} exp(z_j) v_j / sum exp(z_j)
        part_lse = log sum_{j in p, visible} exp(z_j)
    and 0 / -inf where partition p holds no visible key."""
    qf = bf16_bits_to_f64(q)
    B, T, Hq, D = qf.shape
    P = num_partitions
    part_out = np.zeros((B, T, Hq, P, D), dtype=np.float64)
    part_lse = np.full((B, T, Hq, P), -np.inf, dtype=np.float64)
    for s in range(B):
        n = int(context_lens[s])
        if n == 0:
            continue
        if n < T:
            part_out[s] = np.nan
            part_lse[s] = np.nan
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], n)
        vis = causal_visible(n - T, T)
        for t in range(T):
            for p in range(P):
                lo, hi = p * partition_size, min(int(vis[t]), (p + 1) * partition_size)
                if lo >= hi:
                    continue
                for h in range(Hq):
                    g = kv_head_of(h, Hq, num_kv_heads)
                    z = scores(qf[s, t, h, :][None, :], K[lo:hi, g, :], scale)[0]
                    m = np.max(z)
                    e = np.exp(z - m)
                    part_out[s, t, h, p] = (e @ V[lo:hi, g, :]) / np.sum(e)
                    part_lse[s, t, h, p] = m + np.log(np.sum(e))
    return part_out, part_lse


def copy_blocks(dst_k, dst_v, dst_ids, src_k, src_v, src_ids, num_copies):
    """Block-granular KV copy.  For i in [0, num_copies): destination block
    dst_ids[i] (block i when dst_ids is None) receives source block
    src_ids[i] (block i when src_ids is None) -- the whole [Hkv, D/W, 16, W]
    K tile and [Hkv, D, 16] V tile, bit for bit.  A copy whose source or
    destination id lies outside its pool is skipped.  Returns new destination
    pools (uint16 bit patterns)."""
    dk = np.array(dst_k, copy=True)
    dv = np.array(dst_v, copy=True)
    for i in range(num_copies):
        s = i if src_ids is None else int(src_ids[i])
        d = i if dst_ids is None else int(dst_ids[i])
        if not (0 <= s < src_k.shape[0] and 0 <= d < dk.shape[0]):
            continue
        dk[d] = src_k[s]
        dv[d] = src_v[s]
    return dk, dv
