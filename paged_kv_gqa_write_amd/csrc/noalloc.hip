// pa_decode_noalloc: pa_decode + pa_decode_reduce with the split-K pieces
// kept in a static device array instead of a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// `scratch` is a file-scope device array: every GPU the library runs on gets
// its own copy, at its own address, held until the process ends.  In host
// code the array's name is only a host-side stand-in, so the device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever handed to a kernel.  Every call on
// a GPU shares that GPU's array: calls that overlap on one GPU race.  The
// decode kernel writes every piece of the launch before the reduce reads
// it, so nothing in the array has to start at zero (no clearing, no
// memset).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pa.h"
#include "pa_launch.h"

namespace {

// 16 MiB per device: the partial outputs [B, Hq, P, D] fp32 followed by the
// LSEs [B, Hq, P] fp32 (e.g. batch 8 x 16 heads x 20 partitions x head_dim
// 256 takes 2.6 MiB; batch 4 x 64 heads x 8 partitions x 128, 1 MiB).
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of the current device's scratch array, or nullptr.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t partition_size,
                                 int32_t num_partitions, float scale, void* stream) {
  const int st = pa::validate_decode(num_seqs, 1, num_q_heads, num_kv_heads, head_dim,
                                     block_size, num_blocks, max_blocks_per_seq, partition_size,
                                     num_partitions, scale);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (num_partitions == 1)  // no pieces: the decode kernel writes `out` itself
    return pa::launch_decode(out, nullptr, nullptr, q, k_cache, v_cache, block_tables,
                             context_lens, nullptr, nullptr, num_seqs, 1, num_q_heads,
                             num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                             partition_size, 1, scale, s);
  // Pieces, then LSEs at the next 256-byte boundary.
  const uint64_t pieces = (uint64_t)num_seqs * num_q_heads * num_partitions;
  const uint64_t out_bytes = (pieces * head_dim * sizeof(float) + 255) / 256 * 256;
  if (out_bytes + pieces * sizeof(float) > kScratchBytes) return PA_ERR_TOO_LARGE;
  char* base = static_cast<char*>(device_scratch());
  if (base == nullptr) return PA_ERR_LAUNCH;
  float* part_out = reinterpret_cast<float*>(base);
  float* part_lse = reinterpret_cast<float*>(base + out_bytes);
  int rc = pa::launch_decode(nullptr, part_out, part_lse, q, k_cache, v_cache, block_tables,
                             context_lens, nullptr, nullptr, num_seqs, 1, num_q_heads,
                             num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                             partition_size, num_partitions, scale, s);
  if (rc != 0) return rc;
  return pa::launch_decode_reduce(out, part_out, part_lse, context_lens, num_seqs, 1,
                                  num_q_heads, head_dim, partition_size, num_partitions, s);
}
