// C ABI of the paged GQA attention library: host-side argument validation,
// then a launch on the caller's stream.  Nothing here allocates, frees or
// synchronises.  Every check happens before any HIP call, so an invalid call
// returns without touching the device.
#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "pa.h"
#include "pa_launch.h"

namespace {

constexpr int kBlockSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxQueryLen = 16;
constexpr int64_t kMaxGrid = 0x7FFFFFFF;

bool supported_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }

int check_heads(int32_t hq, int32_t hkv, int32_t d, int32_t bs) {
  if (hq <= 0 || hkv <= 0) return PA_ERR_INVALID_ARG;
  if (hq % hkv != 0) return PA_ERR_INVALID_ARG;
  if (hq / hkv > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(d)) return PA_ERR_UNSUPPORTED;
  if (bs != kBlockSize) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// The kernels index positions and blocks inside the partitions' cover
// (num_partitions * partition_size tokens, plus up to one 32-key pair past
// its end) with 32-bit integers.
bool covers_in_int32(int32_t partition_size, int32_t num_partitions) {
  return (int64_t)partition_size * num_partitions <= 0x7FFFFFFFLL - 64;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// The address under which the kernels may access a caller's buffer: device
// memory of the current device as it is, pinned host memory through its
// device mapping.  Pageable host memory, another device's memory and
// unknown pointers are rejected, so no kernel is ever handed an address it
// cannot reach.  A failed query leaves an error in HIP's last-error slot;
// it is cleared so that it cannot surface from a later, unrelated call.
int device_address(const void* p, const void** out) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_INVALID_ARG;
  }
  if (a.type == hipMemoryTypeDevice) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != a.device) {
      (void)hipGetLastError();
      return PA_ERR_INVALID_ARG;
    }
    *out = p;
    return PA_OK;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer != nullptr && a.hostPointer != nullptr) {
    // Offset of p inside the mapping, whether the query reports the
    // mapping's base or p itself.
    const char* host = static_cast<const char*>(a.hostPointer);
    *out = static_cast<const char*>(a.devicePointer) + (static_cast<const char*>(p) - host);
    return PA_OK;
  }
  return PA_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

int pa_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                void* k_cache, void* v_cache, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int64_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim) || block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
  return pa::launch_write_kv(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens,
                             num_kv_heads, head_dim, num_blocks, as_stream(stream));
}

}  // extern "C"

namespace pa {

int validate_decode(int32_t num_seqs, int32_t query_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t max_blocks_per_seq, int32_t partition_size,
                    int32_t num_partitions, float scale) {
  if (num_seqs < 0 || num_blocks < 0) return PA_ERR_INVALID_ARG;
  if (query_len < 1) return PA_ERR_INVALID_ARG;
  if (query_len > kMaxQueryLen) return PA_ERR_UNSUPPORTED;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (partition_size <= 0 || partition_size % kBlockSize != 0) return PA_ERR_INVALID_ARG;
  if (num_partitions < 1) return PA_ERR_INVALID_ARG;
  if (!covers_in_int32(partition_size, num_partitions)) return PA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || scale < 0.f) return PA_ERR_INVALID_ARG;
  // Launch size (one workgroup per 32 columns of a partition) and the
  // number of output rows both index with 32-bit integers.
  const int64_t chunks = ((int64_t)query_len * (num_q_heads / num_kv_heads) + 31) / 32;
  if ((int64_t)num_partitions * num_kv_heads * num_seqs * chunks > kMaxGrid)
    return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * query_len * num_q_heads > kMaxGrid) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

}  // namespace pa

extern "C" {

int pa_decode_multi(void* out, float* part_out, float* part_lse, const void* q,
                    const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t query_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t partition_size, int32_t num_partitions, float scale, void* stream) {
  const int st = pa::validate_decode(num_seqs, query_len, num_q_heads, num_kv_heads, head_dim,
                                     block_size, num_blocks, max_blocks_per_seq, partition_size,
                                     num_partitions, scale);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (num_partitions == 1 && !out) return PA_ERR_INVALID_ARG;
  if (num_partitions > 1 && (!part_out || !part_lse)) return PA_ERR_INVALID_ARG;
  return pa::launch_decode(out, part_out, part_lse, q, k_cache, v_cache, block_tables,
                           context_lens, nullptr, nullptr, num_seqs, query_len, num_q_heads,
                           num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                           partition_size, num_partitions, scale, as_stream(stream));
}

int pa_decode_append(void* out, float* part_out, float* part_lse, const void* q,
                     const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int64_t num_blocks,
                     int32_t max_blocks_per_seq, int32_t partition_size,
                     int32_t num_partitions, float scale, void* stream) {
  if (num_seqs < 0 || num_blocks < 0) return PA_ERR_INVALID_ARG;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (partition_size <= 0 || partition_size % kBlockSize != 0) return PA_ERR_INVALID_ARG;
  if (num_partitions < 1) return PA_ERR_INVALID_ARG;
  if (!covers_in_int32(partition_size, num_partitions)) return PA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || scale < 0.f) return PA_ERR_INVALID_ARG;
  if ((int64_t)num_partitions * num_kv_heads * num_seqs > kMaxGrid) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * num_q_heads > kMaxGrid) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (num_partitions == 1 && !out) return PA_ERR_INVALID_ARG;
  if (num_partitions > 1 && (!part_out || !part_lse)) return PA_ERR_INVALID_ARG;
  return pa::launch_decode(out, part_out, part_lse, q, k_cache, v_cache, block_tables,
                           context_lens, k_new, v_new, num_seqs, 1, num_q_heads, num_kv_heads,
                           head_dim, num_blocks, max_blocks_per_seq, partition_size,
                           num_partitions, scale, as_stream(stream));
}

int pa_decode(void* out, float* part_out, float* part_lse, const void* q, const void* k_cache,
              const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
              int32_t partition_size, int32_t num_partitions, float scale, void* stream) {
  return pa_decode_multi(out, part_out, part_lse, q, k_cache, v_cache, block_tables,
                         context_lens, num_seqs, 1, num_q_heads, num_kv_heads, head_dim,
                         block_size, num_blocks, max_blocks_per_seq, partition_size,
                         num_partitions, scale, stream);
}

int pa_decode_multi_reduce(void* out, const float* part_out, const float* part_lse,
                           const int32_t* context_lens, int32_t num_seqs, int32_t query_len,
                           int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                           int32_t num_partitions, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0) return PA_ERR_INVALID_ARG;
  if (query_len < 1) return PA_ERR_INVALID_ARG;
  if (query_len > kMaxQueryLen) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (partition_size <= 0 || partition_size % kBlockSize != 0) return PA_ERR_INVALID_ARG;
  if (num_partitions < 1) return PA_ERR_INVALID_ARG;
  if (!covers_in_int32(partition_size, num_partitions)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)query_len * num_q_heads > kMaxGrid) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * query_len * num_q_heads > kMaxGrid) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !part_out || !part_lse) return PA_ERR_INVALID_ARG;
  return pa::launch_decode_reduce(out, part_out, part_lse, context_lens, num_seqs, query_len,
                                  num_q_heads, head_dim, partition_size, num_partitions,
                                  as_stream(stream));
}

int pa_decode_reduce(void* out, const float* part_out, const float* part_lse,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t head_dim, int32_t partition_size, int32_t num_partitions,
                     void* stream) {
  return pa_decode_multi_reduce(out, part_out, part_lse, context_lens, num_seqs, 1, num_q_heads,
                                head_dim, partition_size, num_partitions, stream);
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* cu_seqlens,
               const int32_t* prefix_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
               int64_t num_blocks, int32_t max_blocks_per_seq, float scale, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_blocks < 0) return PA_ERR_INVALID_ARG;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PA_OK) return st;
  // The kernel forms a block's element offset as a 32-bit product.
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !cu_seqlens)
    return PA_ERR_INVALID_ARG;
  return pa::launch_prefill(out, q, k_cache, v_cache, block_tables, cu_seqlens, prefix_lens,
                            num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                            num_blocks, max_blocks_per_seq, scale, as_stream(stream));
}

int pa_copy_blocks(void* dst_k_cache, void* dst_v_cache, int64_t dst_num_blocks,
                   const int32_t* dst_block_ids, const void* src_k_cache,
                   const void* src_v_cache, int64_t src_num_blocks,
                   const int32_t* src_block_ids, int32_t num_copies, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, void* stream) {
  if (num_copies < 0 || num_kv_heads <= 0 || dst_num_blocks < 0 || src_num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim) || block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (2 * (int64_t)num_copies > kMaxGrid) return PA_ERR_UNSUPPORTED;
  if (num_copies == 0) return PA_OK;
  if (!dst_k_cache || !dst_v_cache || !src_k_cache || !src_v_cache) return PA_ERR_INVALID_ARG;
  const void* bufs[4] = {dst_k_cache, dst_v_cache, src_k_cache, src_v_cache};
  for (const void* b : bufs)
    if (reinterpret_cast<uintptr_t>(b) % 16 != 0) return PA_ERR_INVALID_ARG;
  const void *dk, *dv, *sk, *sv, *di = nullptr, *si = nullptr;
  int st;
  if ((st = device_address(dst_k_cache, &dk)) != PA_OK) return st;
  if ((st = device_address(dst_v_cache, &dv)) != PA_OK) return st;
  if ((st = device_address(src_k_cache, &sk)) != PA_OK) return st;
  if ((st = device_address(src_v_cache, &sv)) != PA_OK) return st;
  if (dst_block_ids && (st = device_address(dst_block_ids, &di)) != PA_OK) return st;
  if (src_block_ids && (st = device_address(src_block_ids, &si)) != PA_OK) return st;
  return pa::launch_copy_blocks(const_cast<void*>(dk), const_cast<void*>(dv), dst_num_blocks,
                                static_cast<const int32_t*>(di), sk, sv, src_num_blocks,
                                static_cast<const int32_t*>(si), num_copies, num_kv_heads,
                                head_dim, as_stream(stream));
}

int pa_decode_split_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                         int32_t num_compute_units, int32_t* partition_size,
                         int32_t* num_partitions) {
  if (!partition_size || !num_partitions) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0 || num_compute_units <= 0)
    return PA_ERR_INVALID_ARG;
  // The decode kernel is latency-bound when a launch is small, so aim for
  // one workgroup per CU: split each (sequence, KV head) into enough
  // partitions, but never below 4 pairs of blocks (at least one 32-key pair
  // per wave of a 3- or 4-wave workgroup).
  // Partitions are whole pairs (multiples of 32 tokens); the waves of a
  // workgroup split a partition's pairs evenly.
  constexpr int64_t kPair = 32;
  constexpr int64_t kMinPart = 4 * kPair;
  const int64_t items = (int64_t)num_seqs * num_kv_heads;
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  int64_t parts = items > 0 ? (num_compute_units + items - 1) / items : 1;
  const int64_t max_parts = (ctx + kMinPart - 1) / kMinPart;
  if (parts > max_parts) parts = max_parts;
  if (parts < 1) parts = 1;
  int64_t ps = (ctx + parts - 1) / parts;
  ps = ((ps + kPair - 1) / kPair) * kPair;
  int64_t np = (ctx + ps - 1) / ps;
  if (np == 1) ps = ((ctx + kBlockSize - 1) / kBlockSize) * kBlockSize;
  if (ps > 0x7FFFFFF0LL) return PA_ERR_INVALID_ARG;
  *partition_size = (int32_t)ps;
  *num_partitions = (int32_t)np;
  return PA_OK;
}

int pa_decode_split_plan_lens(int32_t num_seqs, int32_t num_kv_heads,
                              const int32_t* context_lens, int32_t num_compute_units,
                              int32_t* partition_size, int32_t* num_partitions) {
  if (!partition_size || !num_partitions) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_kv_heads <= 0 || num_compute_units <= 0) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && !context_lens) return PA_ERR_INVALID_ARG;
  int64_t max_ctx = 0;
  for (int32_t s = 0; s < num_seqs; ++s) max_ctx = std::max<int64_t>(max_ctx, context_lens[s]);
  // Beyond 64 sequences the decode kernel keeps the plain launch order, in
  // which empty workgroups may sit ahead of live ones: plan from the longest.
  if (num_seqs > 64)
    return pa_decode_split_plan(num_seqs, num_kv_heads, (int32_t)max_ctx, num_compute_units,
                                partition_size, num_partitions);
  // A launch holds one workgroup per (partition, KV head, sequence); with up
  // to 64 sequences the decode kernel ranks the ones whose partition holds
  // keys first, and the empty ones (past their sequence's length) after them.
  // The longest workgroup sets the launch time, so take the smallest
  // partition (whole 32-key pairs, at least 4 of them) whose live
  // workgroups still fit one per compute unit, counted over the actual
  // lengths: a batch mixing short and long contexts then gives its long
  // sequences more partitions instead of leaving compute units idle.
  constexpr int64_t kPair = 32;
  constexpr int64_t kMinPart = 4 * kPair;
  const int64_t ctx = max_ctx > 0 ? max_ctx : 1;
  auto live = [&](int64_t ps) {
    int64_t n = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
      if (context_lens[s] > 0) n += ((int64_t)context_lens[s] + ps - 1) / ps;
    return n * num_kv_heads;
  };
  const int64_t whole = ((ctx + kBlockSize - 1) / kBlockSize) * kBlockSize;
  int64_t ps = whole, np = 1;
  const int64_t k_hi = (ctx + kPair - 1) / kPair;  // ps = 32*k_hi covers ctx in one piece
  if (k_hi > kMinPart / kPair && live(kPair * k_hi) < num_compute_units) {
    // One piece per sequence leaves compute units idle.  live() does not
    // increase with ps: find the smallest k >= 4 with live(32k) <= CUs
    // (k_hi satisfies it).
    int64_t lo = kMinPart / kPair, hi = k_hi;  // invariant: live(32*hi) <= CUs
    if (live(kPair * lo) <= num_compute_units) hi = lo;
    while (hi - lo > 1) {  // invariant: live(32*lo) > CUs
      const int64_t mid = (lo + hi) / 2;
      if (live(kPair * mid) <= num_compute_units) hi = mid;
      else lo = mid;
    }
    ps = kPair * hi;
    np = (ctx + ps - 1) / ps;
    if (np == 1) ps = whole;
  }
  // A workgroup's time follows its partition's length in whole pairs per
  // wave, while a launch beyond one dispatch round pays for the ranking (a
  // second round trip before the K/V stream): keep the plan from the longest
  // context unless the lengths allow a substantially shorter partition.
  int32_t max_ps = 0, max_np = 0;
  const int rc = pa_decode_split_plan(num_seqs, num_kv_heads, (int32_t)max_ctx,
                                      num_compute_units, &max_ps, &max_np);
  if (rc != PA_OK) return rc;
  if (3 * ps > 2 * (int64_t)max_ps) {
    ps = max_ps;
    np = max_np;
  }
  if (ps > 0x7FFFFFF0LL) return PA_ERR_INVALID_ARG;
  *partition_size = (int32_t)ps;
  *num_partitions = (int32_t)np;
  return PA_OK;
}

int pa_decode_multi_split_plan(int32_t num_seqs, int32_t query_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t max_context_len,
                               int32_t num_compute_units, int32_t* partition_size,
                               int32_t* num_partitions) {
  if (!partition_size || !num_partitions) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || query_len < 1 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || max_context_len < 0 || num_compute_units <= 0)
    return PA_ERR_INVALID_ARG;
  // Workgroups of a launch with P partitions, as pa_decode_multi makes them:
  // items = P x KV heads x sequences; T*G columns in tiles of 16; two tiles
  // per wave once items x ceil(tiles/2) fill the CUs, else one tile per
  // workgroup (a workgroup per tile).  The plan takes the most partitions
  // whose launch still fits in one workgroup per CU (more than that adds a
  // second dispatch round), in whole 32-key pairs and at least 4 pairs each.
  constexpr int64_t kPair = 32;
  constexpr int64_t kMinPart = 4 * kPair;
  const int64_t tiles = ((int64_t)query_len * (num_q_heads / num_kv_heads) + 15) / 16;
  const int64_t base = (int64_t)num_seqs * num_kv_heads;
  const int64_t cus = num_compute_units;
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  auto shape = [&](int64_t parts, int64_t& ps, int64_t& np) {
    ps = (ctx + parts - 1) / parts;
    ps = ((ps + kPair - 1) / kPair) * kPair;
    np = (ctx + ps - 1) / ps;
    if (np == 1) ps = ((ctx + kBlockSize - 1) / kBlockSize) * kBlockSize;
  };
  auto workgroups = [&](int64_t np) {
    const int64_t items = base * np;
    const bool two = tiles >= 2 && items * ((tiles + 1) / 2) >= cus;
    return items * (two ? (tiles + 1) / 2 : tiles);
  };
  int64_t best_ps = 0, best_np = 0;
  shape(1, best_ps, best_np);
  const int64_t max_parts = std::min<int64_t>((ctx + kMinPart - 1) / kMinPart, cus);
  for (int64_t parts = 2; parts <= max_parts && base > 0; ++parts) {
    int64_t ps, np;
    shape(parts, ps, np);
    if (np > best_np && workgroups(np) <= cus) {
      best_ps = ps;
      best_np = np;
    }
  }
  if (best_ps > 0x7FFFFFF0LL) return PA_ERR_INVALID_ARG;
  *partition_size = (int32_t)best_ps;
  *num_partitions = (int32_t)best_np;
  return PA_OK;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: unsupported shape";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: kernel launch failed";
    case PA_ERR_NO_MEMORY: return "PA_ERR_NO_MEMORY: host allocation failed";
    case PA_ERR_TOO_LARGE:
      return "PA_ERR_TOO_LARGE: split-K pieces exceed the library's static scratch";
    default: return "unknown pa_status";
  }
}

}  // extern "C"
