// Block-granular KV copy: whole (block, all KV heads) tiles of the K and V
// pools move from a source to a destination, each side being a pool
// addressed by block ids or a packed run of blocks.  Restoring sealed blocks
// from a host tier, saving them to it and duplicating a shared block inside
// one pool are all this copy; either side may live in device memory or in
// pinned host memory (the kernel then reads or writes it over the host link
// directly, with no staging pass through HBM).
//
// One workgroup per (copy, K or V): it streams the block's Hkv*16*D bf16
// values as 16-byte vectors, KUNROLL loads in flight per lane before the
// matching stores.  Block ids are wave-uniform scalar loads.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    u32x4* __restrict__ dst_k, u32x4* __restrict__ dst_v, int64_t dst_num_blocks,
    const int32_t* __restrict__ dst_ids, const u32x4* __restrict__ src_k,
    const u32x4* __restrict__ src_v, int64_t src_num_blocks, const int32_t* __restrict__ src_ids,
    int vecs_per_block) {
  const int i = blockIdx.x >> 1;
  const bool is_v = (blockIdx.x & 1) != 0;
  const int64_t s = src_ids != nullptr ? (int64_t)src_ids[i] : i;
  const int64_t d = dst_ids != nullptr ? (int64_t)dst_ids[i] : i;
  if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks) return;
  const u32x4* src = (is_v ? src_v : src_k) + s * vecs_per_block;
  u32x4* dst = (is_v ? dst_v : dst_k) + d * vecs_per_block;
  for (int base = threadIdx.x; base < vecs_per_block; base += kCopyThreads * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = base + u * kCopyThreads;
      if (j < vecs_per_block) r[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = base + u * kCopyThreads;
      if (j < vecs_per_block) dst[j] = r[u];
    }
  }
}

}  // namespace

int launch_copy_blocks(void* dst_k, void* dst_v, int64_t dst_num_blocks, const int32_t* dst_ids,
                       const void* src_k, const void* src_v, int64_t src_num_blocks,
                       const int32_t* src_ids, int num_copies, int num_kv_heads, int head_dim,
                       hipStream_t stream) {
  // One block of one pool holds Hkv * 16 * D bf16 values = Hkv * D * 2
  // sixteen-byte vectors.
  const int vecs = num_kv_heads * head_dim * 2;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(2u * (unsigned)num_copies), dim3(kCopyThreads), 0,
                     stream, (u32x4*)dst_k, (u32x4*)dst_v, dst_num_blocks, dst_ids,
                     (const u32x4*)src_k, (const u32x4*)src_v, src_num_blocks, src_ids, vecs);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pa
