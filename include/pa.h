/*
 * pa.h -- grouped-query attention over a paged KV cache, for AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers (device memory unless a call says
 * otherwise), sizes and an opaque HIP stream handle; no framework types.
 *
 * What the operations compute comes from the serving pages this library
 * follows ("Qwen3-4B / 8B / 32B", section Architecture Notes; "Qwen3.5-4B /
 * 9B / 27B" and "Qwen3.5 Dense" for the hybrid models' full-attention
 * layers):
 *   - full attention with grouped-query attention: Hq query heads share Hkv
 *     KV heads (32/8 for Qwen3-4B, group 8 for Qwen3-32B); query head h reads
 *     KV head h / (Hq/Hkv);
 *   - a paged KV cache with full-lifetime admission (a sequence's block-table
 *     row may already list blocks past its current length; those entries are
 *     never read);
 *   - prefix caching on by default: a prefill attends to cached prefix blocks
 *     and computes only the new tokens ("Qwen3-4B / 8B / 32B", section Warm
 *     Prefix-Cache TTFT).
 * Attention is scaled dot-product softmax attention,
 *   out = sum_j exp(z_j) v_j / sum_j exp(z_j),   z_j = scale * <q, k_j>,
 * computed with fp32 accumulation and bf16 inputs/outputs.
 *
 * ---------------------------------------------------------------------------
 * Memory layout (all tensors row-major and contiguous; bf16 = 16-bit storage)
 * ---------------------------------------------------------------------------
 *   block_size (BS) is 16 tokens.
 *   K pool   [num_blocks, Hkv, D/32, 16, 32]  bf16: the head dimension is
 *            cut into 32-wide slices and each slice holds the block's 16
 *            keys as 64-byte rows -- element d of the K row of the token at
 *            in-block offset o of block b for KV head g is at
 *            (((b*Hkv+g)*(D/32) + d/32)*16 + o)*32 + d%32.
 *   V pool   [num_blocks, Hkv, D, 16]  bf16: "transposed" -- element d of
 *            that token's V row is at ((b*Hkv+g)*D+d)*16+o.  Each (block,
 *            head) of either pool is one contiguous 16*D*2-byte tile.
 *   slot     b*16 + o names a token's place in the pools.
 *   block_tables [num_seqs, max_blocks_per_seq] int32: logical block i of
 *            sequence s (positions 16i..16i+15) is physical block
 *            block_tables[s*max_blocks_per_seq + i].
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every call
 * ---------------------------------------------------------------------------
 *   Ownership: the caller allocates and owns every buffer, including the
 *     split-K workspace.  The GPU calls never allocate, free or
 *     synchronise; each only enqueues kernels on `stream` (a hipStream_t
 *     passed as void*; NULL = the default stream), so they are asynchronous,
 *     stateless, thread-safe and may be captured in a HIP graph.  The
 *     host-side prefix index (pa_prefix_index_*) is the one stateful object:
 *     it owns the host memory it allocates and runs on the CPU only.
 *   Errors: arguments are checked on the host before anything is enqueued;
 *     on failure the call returns a negative pa_status and writes nothing.
 *     A failed kernel launch returns PA_ERR_LAUNCH.
 *   Device-side data (table entries, lengths, slots) is validated by the
 *     kernels without ever addressing memory outside the buffers described by
 *     the size arguments: a block-table entry outside [0, num_blocks) that a
 *     live position needs, a length that exceeds max_blocks_per_seq*16, or a
 *     decode context longer than partition_size*num_partitions makes the
 *     affected sequence's outputs NaN (and its split-K LSEs NaN).  So does a
 *     negative context length, in every call that reads one (the reduces
 *     included).  The product num_partitions*partition_size must stay below
 *     2^31 - 64 (PA_ERR_UNSUPPORTED otherwise).
 *   Supported shapes: head_dim in {64, 128, 256}; num_q_heads a multiple of
 *     num_kv_heads with a group Hq/Hkv of at most 16; block_size == 16;
 *     num_kv_heads at most 65535 for pa_write_kv, pa_copy_blocks and
 *     pa_prefill (PA_ERR_UNSUPPORTED otherwise).
 *   Sizes of 0 (no tokens, no sequences) are valid no-ops.
 */
#ifndef PAGED_KV_GQA_PA_H
#define PAGED_KV_GQA_PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null pointer, negative size, inconsistent sizes */
  PA_ERR_UNSUPPORTED = -2,  /* head_dim / group / block_size outside the supported set */
  PA_ERR_LAUNCH = -3,       /* the HIP runtime rejected a kernel launch */
  PA_ERR_NO_MEMORY = -4,    /* host allocation failed (prefix index only) */
  PA_ERR_TOO_LARGE = -5     /* split-K pieces exceed the static scratch (pa_decode_noalloc) */
} pa_status;

/*
 * pa_write_kv -- slot-mapped KV append (the write side of the paged KV cache,
 * "Qwen3-4B / 8B / 32B", Architecture Notes).
 *
 * For every token t in [0, num_tokens) with slot = slot_mapping[t] >= 0:
 *   K row of (slot/16, head g, offset slot%16) := k_new[t, g, :]  (its 64-byte
 *       piece in each of the D/32 slices of the tile, layout above)
 *   V pool column of (slot/16, head g, offset slot%16) := v_new[t, g, :]
 * for all KV heads g.  Pure bit copies (bit-exact).  Slots < 0 are skipped;
 * slots >= num_blocks*16 are invalid and skipped as well (never written).
 * Two tokens naming the same slot race (last writer unspecified).
 *
 *   k_new, v_new   device, bf16 [num_tokens, Hkv, D]
 *   slot_mapping   device, int64 [num_tokens]
 *   k_cache        device, bf16 K pool (layout above), updated in place
 *   v_cache        device, bf16 V pool (layout above), updated in place
 */
int pa_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                void* k_cache, void* v_cache,
                int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, int64_t num_blocks, void* stream);

/*
 * pa_decode -- one query token per sequence attends over its paged context
 * (decode of the full-attention layers; "Qwen3-4B / 8B / 32B", Architecture
 * Notes).  Sequence s's query sits at position context_lens[s]-1 and sees
 * keys 0..context_lens[s]-1 (its own K/V must already be in the pool, e.g.
 * written by pa_write_kv on the same stream).
 *
 * Split-K: the context is cut into partitions of partition_size tokens
 * (partition p covers positions [p*ps, (p+1)*ps)).
 *   num_partitions == 1: writes out[s, h, :] (bf16) directly; part_out and
 *     part_lse are not used and may be NULL.
 *   num_partitions  > 1: writes, for every (s, h, p),
 *       part_out[s, h, p, :] = sum_{j in p} e^{z_j} v_j / sum_{j in p} e^{z_j}
 *       part_lse[s, h, p]    = ln sum_{j in p} e^{z_j}
 *     (fp32; an empty partition gives 0 and -inf); `out` is not touched and
 *     may be NULL.  pa_decode_reduce then produces `out`.
 *   num_partitions*partition_size must cover every context length.
 *
 *   out            device, bf16 [num_seqs, Hq, D]
 *   part_out       device, fp32 [num_seqs, Hq, num_partitions, D]
 *   part_lse       device, fp32 [num_seqs, Hq, num_partitions]
 *   q              device, bf16 [num_seqs, Hq, D]
 *   k_cache, v_cache   device, pools (layout above)
 *   block_tables   device, int32 [num_seqs, max_blocks_per_seq]
 *   context_lens   device, int32 [num_seqs] (0 gives a zero output)
 *   partition_size multiple of 16, > 0
 *   scale          softmax scale applied to <q, k> in fp32 (e.g. 1/sqrt(D));
 *                  finite and >= 0 (a negative scale is PA_ERR_INVALID_ARG)
 */
int pa_decode(void* out, float* part_out, float* part_lse,
              const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens,
              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
              int32_t partition_size, int32_t num_partitions,
              float scale, void* stream);

/*
 * pa_decode_append -- pa_write_kv of each sequence's new token followed by
 * pa_decode, in one kernel: the decode step of the full-attention layers
 * appends the token's K/V to the paged cache and attends over it
 * ("Qwen3-4B / 8B / 32B", Architecture Notes).  For every sequence s with
 * context_lens[s] > 0 the token at position ctx-1 (K/V = k_new[s], v_new[s])
 * is written to the slot the block table gives that position, and the
 * outputs are those pa_decode would produce after that write (bit for bit).
 * The kernel does not read the new token back from the pool, so no
 * ordering between the write and the reads is needed.  A sequence whose
 * table entry for position ctx-1 is outside the pool (or any other invalid
 * entry) gets NaN outputs, and that token is not written.
 *
 *   k_new, v_new   device, bf16 [num_seqs, Hkv, D]
 *   k_cache, v_cache   device, pools, updated in place at the new slots
 *   other arguments as for pa_decode (num_partitions > 1: finish with
 *   pa_decode_reduce).
 */
int pa_decode_append(void* out, float* part_out, float* part_lse,
                     const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int64_t num_blocks,
                     int32_t max_blocks_per_seq, int32_t partition_size,
                     int32_t num_partitions, float scale, void* stream);

/*
 * pa_decode_noalloc -- pa_decode followed (when num_partitions > 1) by
 * pa_decode_reduce, with no workspace argument and no allocation: for
 * callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * split-K pieces live in a static device array of the library (16 MiB per
 * GPU, held until the process ends): B * Hq * num_partitions pieces of
 * D + 1 floats (the pieces rounded up to 256 bytes, then the LSEs) must fit,
 * else PA_ERR_TOO_LARGE and nothing is enqueued.  Every call on a GPU shares
 * that GPU's array, so calls that overlap on one GPU (another stream, another
 * host thread) race; calls on one stream are ordered.  Writes out[s, h, :]
 * (bf16), bit for bit what pa_decode (+ pa_decode_reduce with the same
 * context_lens) writes.  The first call on a device with num_partitions > 1
 * looks up that device's copy of the array (PA_ERR_LAUNCH if that fails).
 *
 *   out            device, bf16 [num_seqs, Hq, D] (required)
 *   other arguments as for pa_decode.
 */
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t partition_size,
                      int32_t num_partitions, float scale, void* stream);

/*
 * pa_decode_reduce -- log-sum-exp combination of pa_decode's split-K pieces:
 *   M = max_p lse_p,  w_p = e^{lse_p - M},
 *   out[s, h, :] = bf16( sum_p w_p part_out[s, h, p, :] / sum_p w_p ),
 * zero when every partition is empty; NaN when any read LSE is NaN.
 *
 *   context_lens   device int32 [num_seqs] or NULL.  When given, only the
 *                  partitions p < ceil(ctx/partition_size) are read (none
 *                  for ctx == 0: zero output; ctx < 0 is invalid: NaN); when
 *                  NULL all num_partitions are read (empty ones must hold
 *                  lse = -inf, as pa_decode writes them).
 *   other arguments as for pa_decode.
 */
int pa_decode_reduce(void* out, const float* part_out, const float* part_lse,
                     const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                     int32_t partition_size, int32_t num_partitions, void* stream);

/*
 * pa_decode_multi -- decode with T = query_len query tokens per sequence:
 * the target-model pass that verifies a block of drafted tokens in
 * speculative decoding ("Qwen3-4B / 8B / 32B", section DSpark Speculative
 * Decoding: a drafter proposes a block of tokens and the target model checks
 * them greedily in one forward pass).  pa_decode is the case T = 1.
 *
 * context_lens[s] counts every cached token of sequence s, including its T
 * query tokens, whose K/V must already be in the pool (e.g. written by
 * pa_write_kv on the same stream).  Query token t (0 <= t < T) sits at
 * position ctx - T + t and attends to keys 0..ctx - T + t: the cached
 * context plus, causally, the query tokens up to itself.  A sequence with
 * context_lens[s] == 0 gets zero outputs; 0 < context_lens[s] < T is
 * invalid and gives NaN outputs for that sequence.
 *
 * Split-K exactly as for pa_decode, one piece per (s, t, h, p):
 *   num_partitions == 1: writes out[s, t, h, :] (bf16); part_out/part_lse
 *     unused (may be NULL).
 *   num_partitions  > 1: writes
 *       part_out[s, t, h, p, :] = sum_{j in p, j visible to t} e^{z_j} v_j / sum e^{z_j}
 *       part_lse[s, t, h, p]    = ln sum_{j in p, j visible to t} e^{z_j}
 *     (0 and -inf where no key of p is visible to t); `out` is not touched.
 *     pa_decode_multi_reduce then produces `out`.
 *
 *   out            device, bf16 [num_seqs, T, Hq, D]
 *   part_out       device, fp32 [num_seqs, T, Hq, num_partitions, D]
 *   part_lse       device, fp32 [num_seqs, T, Hq, num_partitions]
 *   q              device, bf16 [num_seqs, T, Hq, D]
 *   query_len      T, 1..16 (larger: PA_ERR_UNSUPPORTED)
 *   other arguments as for pa_decode.
 */
int pa_decode_multi(void* out, float* part_out, float* part_lse,
                    const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t query_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t partition_size, int32_t num_partitions,
                    float scale, void* stream);

/*
 * pa_decode_multi_reduce -- pa_decode_reduce for pa_decode_multi's pieces:
 * combines part_out[s, t, h, :, :] / part_lse[s, t, h, :] into
 * out[s, t, h, :] (bf16 [num_seqs, T, Hq, D]) with the same formula, zero
 * and NaN rules.  context_lens (or NULL) as for pa_decode_reduce: when given,
 * partitions p < ceil(ctx/partition_size) of every token are read.
 * pa_decode_reduce is the case T = 1.
 */
int pa_decode_multi_reduce(void* out, const float* part_out, const float* part_lse,
                           const int32_t* context_lens, int32_t num_seqs, int32_t query_len,
                           int32_t num_q_heads, int32_t head_dim,
                           int32_t partition_size, int32_t num_partitions, void* stream);

/*
 * pa_prefill -- varlen causal prefill over the paged cache with cached
 * prefixes ("Qwen3-4B / 8B / 32B", sections Warm Prefix-Cache TTFT and
 * Architecture Notes: prefix cache on by default).
 *
 * Sequence s has n_s = cu_seqlens[s+1]-cu_seqlens[s] new tokens following
 * p_s = prefix_lens[s] cached ones.  New token i (packed row cu_seqlens[s]+i)
 * sits at position p_s+i and attends to keys 0..p_s+i, all read through the
 * block table (the new tokens' K/V must already be in the pool).
 *
 *   out            device, bf16 [total_q, Hq, D]
 *   q              device, bf16 [total_q, Hq, D] (packed varlen)
 *   k_cache, v_cache   device, pools (layout above)
 *   block_tables   device, int32 [num_seqs, max_blocks_per_seq]
 *   cu_seqlens     device, int32 [num_seqs+1], non-decreasing, from 0 to
 *                  total_q (rows of a sequence whose range leaves
 *                  [0, total_q] are not written)
 *   prefix_lens    device, int32 [num_seqs], or NULL for no cached prefixes
 *   max_q_len      host upper bound of n_s (sizes the launch grid; rows of
 *                  a sequence beyond it are not written)
 *   scale          as for pa_decode (finite, >= 0)
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* cu_seqlens,
               const int32_t* prefix_lens,
               int32_t num_seqs, int32_t total_q, int32_t max_q_len,
               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
               float scale, void* stream);

/*
 * pa_copy_blocks -- block-granular KV copy: restoring sealed blocks from a
 * host tier instead of recomputing their prefill, saving them to it
 * ("Qwen3-4B / 8B / 32B", section KV Offload), and duplicating a shared
 * block inside one pool.
 *
 * For every i in [0, num_copies):
 *   destination block dst_block_ids[i] := source block src_block_ids[i]
 * for both pools (the whole [Hkv, D/32, 16, 32] K tile and [Hkv, D, 16] V tile,
 * bit for bit).  A NULL id array means "block i" for copy i, i.e. a packed
 * run of num_copies blocks in the pool layout.  A copy whose source id is
 * outside [0, src_num_blocks) or whose destination id is outside
 * [0, dst_num_blocks) is skipped.  Two copies with the same destination
 * race; a block that is both a source and a destination in one call gives
 * an unspecified result.
 *
 *   dst_k_cache, dst_v_cache   destination pools [dst_num_blocks, ...]: device
 *                  memory of the current device or pinned host memory
 *                  (hipHostMalloc); 16-byte aligned
 *   src_k_cache, src_v_cache   source pools [src_num_blocks, ...], same rules
 *   dst_block_ids, src_block_ids   int32 [num_copies] in device or pinned
 *                  host memory, or NULL
 * Pinned host memory is read or written by the kernel over the host link
 * through its device mapping (no staging copy).  Pageable host memory or
 * another device's memory is PA_ERR_INVALID_ARG (checked on the host before
 * anything is enqueued).
 */
int pa_copy_blocks(void* dst_k_cache, void* dst_v_cache, int64_t dst_num_blocks,
                   const int32_t* dst_block_ids,
                   const void* src_k_cache, const void* src_v_cache, int64_t src_num_blocks,
                   const int32_t* src_block_ids,
                   int32_t num_copies, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, void* stream);

/*
 * pa_decode_split_plan -- host-only helper: a partition size (multiple of
 * 16) and count for pa_decode that give the GPU enough independent work
 * items while covering max_context_len.  Writes *partition_size and
 * *num_partitions; returns PA_OK or PA_ERR_INVALID_ARG.
 */
int pa_decode_split_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                         int32_t num_compute_units,
                         int32_t* partition_size, int32_t* num_partitions);

/*
 * pa_decode_split_plan_lens -- host-only helper: the same plan from the
 * batch's actual context lengths (context_lens: HOST int32 [num_seqs], may
 * be NULL when num_seqs == 0).  pa_decode launches one workgroup per
 * (partition, KV head, sequence); with up to 64 sequences it launches those
 * whose partition holds keys first and the empty ones (past their
 * sequence's length) last.  The plan takes the smallest partition (whole
 * 32-key pairs, at least 128 keys) whose live workgroups number at most
 * num_compute_units, so that in a batch of mixed lengths the long sequences
 * get more partitions; when one partition per sequence already gives at
 * least num_compute_units live workgroups, one partition of the longest
 * context (rounded up to 16).  That plan is taken only when its partition
 * is at most 2/3 of the one pa_decode_split_plan gives for the longest
 * context (a launch of more than one workgroup per compute unit pays one
 * extra memory round trip for the ranking); otherwise, and for more than 64
 * sequences, the result is pa_decode_split_plan's.  Writes *partition_size
 * (multiple of 16) and *num_partitions, covering the longest context;
 * returns PA_OK or PA_ERR_INVALID_ARG.
 */
int pa_decode_split_plan_lens(int32_t num_seqs, int32_t num_kv_heads,
                              const int32_t* context_lens, int32_t num_compute_units,
                              int32_t* partition_size, int32_t* num_partitions);

/*
 * pa_decode_multi_split_plan -- host-only helper: partition size and count
 * for pa_decode_multi with T = query_len tokens per sequence.  Its columns
 * (token, query head) come in 16-wide tiles that may be spread over several
 * workgroups, so the plan counts workgroups the way pa_decode_multi launches
 * them and takes the most partitions (whole 32-key pairs, at least 128 keys
 * each) whose launch holds at most one workgroup per compute unit
 * (pa_decode_split_plan may round up to slightly more).  num_q_heads must be
 * a multiple of num_kv_heads.  Writes *partition_size (multiple of 16) and
 * *num_partitions, covering max_context_len; returns PA_OK or
 * PA_ERR_INVALID_ARG.
 */
int pa_decode_multi_split_plan(int32_t num_seqs, int32_t query_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t max_context_len,
                               int32_t num_compute_units,
                               int32_t* partition_size, int32_t* num_partitions);

/*
 * Prefix-block index (host only, no GPU involved): which physical KV blocks
 * already hold the leading full blocks of a token sequence ("Qwen3-4B / 8B /
 * 32B", Architecture Notes: prefix caching on by default, prefix matching
 * against the GPU KV cache; section Warm Prefix-Cache TTFT).  A hit of m
 * blocks lets pa_prefill start at prefix_len = 16*m with those blocks at the
 * head of the sequence's block-table row.
 *
 * Only sealed (full, 16-token) blocks are indexed, each under the token ids
 * of its whole prefix: block i of a sequence matches only if blocks 0..i-1
 * match too.  Matching compares token ids exactly (hash collisions cannot
 * return another prefix's blocks).  Tokens and block ids are host int32
 * arrays.  The index owns the host memory it allocates (created by
 * pa_prefix_index_create, released by pa_prefix_index_destroy).  Calls that
 * modify an index must not overlap with any other call on it; concurrent
 * pa_prefix_index_match calls are safe.  After PA_ERR_NO_MEMORY an index
 * must only be destroyed.
 */
typedef struct pa_prefix_index pa_prefix_index;

/* New empty index holding at most `capacity` (> 0) blocks; *out = NULL on error. */
int pa_prefix_index_create(int64_t capacity, pa_prefix_index** out);

/* Releases the index (NULL is a no-op). */
void pa_prefix_index_destroy(pa_prefix_index* index);

/* Number of indexed blocks (-1 for NULL). */
int64_t pa_prefix_index_size(const pa_prefix_index* index);

/*
 * Longest cached run of leading full blocks of tokens[0..num_tokens):
 * writes its block ids to block_ids[0..*num_matched) (room for
 * num_tokens/16 ids).  A trailing partial block never matches.
 */
int pa_prefix_index_match(const pa_prefix_index* index, const int32_t* tokens,
                          int32_t num_tokens, int32_t* block_ids, int32_t* num_matched);

/*
 * Registers the sealed blocks of a sequence: full block i of tokens lives in
 * physical block block_ids[i] (i < min(num_tokens/16, num_block_ids)).
 * Blocks whose prefix is already cached keep their first block (the id given
 * for them is ignored).  The rest are added in order until a negative id or
 * a full index.  An id already indexed under another prefix means that
 * block was reused: its old entry and every entry extending it are dropped
 * first.  An id that appears twice among the blocks to add, or that holds
 * one of this sequence's cached blocks, is PA_ERR_INVALID_ARG (nothing
 * changes).  *num_inserted = number of blocks added.
 */
int pa_prefix_index_insert(pa_prefix_index* index, const int32_t* tokens, int32_t num_tokens,
                           const int32_t* block_ids, int32_t num_block_ids,
                           int32_t* num_inserted);

/*
 * Drops the entry of physical block block_id (e.g. when the block is freed)
 * and every entry extending it; *num_removed = entries dropped (0 if the
 * block was not indexed).
 */
int pa_prefix_index_remove(pa_prefix_index* index, int32_t block_id, int32_t* num_removed);

/* Host-only: a static string naming a pa_status value. */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_GQA_PA_H */
