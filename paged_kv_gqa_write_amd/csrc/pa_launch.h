// Internal launcher interface between the C ABI (pa_api.hip) and the kernel
// translation units.  Arguments are already validated by the caller; each
// launcher returns 0, -2 (no kernel instance for the shape) or -3 (launch
// rejected by the runtime).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Host checks shared by the decode entry points (everything except the
// pointer arguments): returns PA_OK or the pa_status to report.
int validate_decode(int32_t num_seqs, int32_t query_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t max_blocks_per_seq, int32_t partition_size,
                    int32_t num_partitions, float scale);

int launch_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                    void* k_cache, void* v_cache, int num_tokens, int num_kv_heads,
                    int head_dim, int64_t num_blocks, hipStream_t stream);

// query_len query tokens per sequence (1 for plain decode).  With k_new /
// v_new non-null (query_len 1 only) the kernel also appends each sequence's
// token at position ctx-1 into the pools through the block table.
int launch_decode(void* out, float* part_out, float* part_lse, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  const int32_t* context_lens, const void* k_new, const void* v_new,
                  int num_seqs, int query_len, int num_q_heads, int num_kv_heads, int head_dim,
                  int64_t num_blocks, int max_blocks_per_seq, int partition_size,
                  int num_partitions, float scale, hipStream_t stream);

int launch_decode_reduce(void* out, const float* part_out, const float* part_lse,
                         const int32_t* context_lens, int num_seqs, int query_len,
                         int num_q_heads, int head_dim, int partition_size, int num_partitions,
                         hipStream_t stream);

int launch_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* cu_seqlens,
                   const int32_t* prefix_lens, int num_seqs, int total_q, int max_q_len,
                   int num_q_heads, int num_kv_heads, int head_dim, int64_t num_blocks,
                   int max_blocks_per_seq, float scale, hipStream_t stream);

// Pointers are device addresses (pinned host memory already translated);
// ids may be null (block i for copy i).
int launch_copy_blocks(void* dst_k, void* dst_v, int64_t dst_num_blocks, const int32_t* dst_ids,
                       const void* src_k, const void* src_v, int64_t src_num_blocks,
                       const int32_t* src_ids, int num_copies, int num_kv_heads, int head_dim,
                       hipStream_t stream);

}  // namespace pa
