// Slot-mapped KV append into the paged pools (bit copies).
//
// One workgroup handles 16 consecutive new tokens of one KV head.  Thread
// (t, j) = (tid / 16, tid % 16) owns token t and the j-th sixteenth of the
// head dimension, so 16 consecutive lanes read one token's contiguous row.
// A sixteenth never straddles a 32-wide slice of the K pool, so each thread's
// K piece is contiguous there too (slice d0/32, row `offset`).  When the 16 tokens fill one block in order (every
// full block of a prefill), the workgroup stages the V rows in LDS and
// stores the block's transposed V^T tile in 16-byte pieces; otherwise each
// V element is stored at its (d, offset) place on its own.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int num_tokens, int num_kv_heads, int64_t num_slots) {
  constexpr int EPT = D / 16;  // elements per thread: 4, 8 or 16
  // The group's V rows, token-major (whole-block case).
  __shared__ __attribute__((aligned(16))) uint16_t vrow[kBlock][D];
  const int lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 16;
  const int g = blockIdx.y;
  // Lanes 0..15 of every wave read the slots of the group's 16 tokens.
  const int tq = t0 + (lane & 15);
  const int64_t qslot = tq < num_tokens ? slot_mapping[tq] : -1;
  const int64_t base = __builtin_amdgcn_readfirstlane((int)(qslot & 0xFFFFFFFF)) |
                       ((int64_t)__builtin_amdgcn_readfirstlane((int)(qslot >> 32)) << 32);
  // Whole-block case: the 16 tokens fill one block, in order.  Every wave
  // evaluates the same 16 slots, so the test is uniform over the workgroup.
  const bool whole = (__ballot(qslot == base + (lane & 15)) & 0xFFFFull) == 0xFFFFull &&
                     base >= 0 && base % kBlock == 0 && base + kBlock <= num_slots;
  // This thread: token tl of the group, elements d0..d0+EPT-1 of its rows, so
  // 16 consecutive lanes cover one token's contiguous row.
  const int tl = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * EPT;
  const int t = t0 + tl;
  const int64_t slot = __shfl(qslot, tl, 64);
  if (!whole && (t >= num_tokens || slot < 0 || slot >= num_slots)) return;
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int64_t src = ((int64_t)t * num_kv_heads + g) * D + d0;
  const int64_t tile = (blk * num_kv_heads + g);

  // K: the piece of the token's row, contiguous in k_new and in its slice
  // of the pool (element d at ((tile*D/32 + d/32)*16 + off)*32 + d%32).
  uint16_t* kdst = k_cache + tile * kBlock * D + (d0 / 32) * 32 * kBlock + off * 32 + (d0 % 32);
  if constexpr (EPT == 4) {
    *reinterpret_cast<u32x2*>(kdst) = *reinterpret_cast<const u32x2*>(k_new + src);
  } else {
#pragma unroll
    for (int e = 0; e < EPT; e += 8)
      *reinterpret_cast<u32x4*>(kdst + e) = *reinterpret_cast<const u32x4*>(k_new + src + e);
  }

  if (whole) {
    // V: rows into LDS, then the block's V^T tile as 16-byte pieces (each d
    // row of the tile is 16 tokens: two pieces of 8).
    if constexpr (EPT == 4) {
      *reinterpret_cast<u32x2*>(&vrow[tl][d0]) = *reinterpret_cast<const u32x2*>(v_new + src);
    } else {
#pragma unroll
      for (int e = 0; e < EPT; e += 8)
        *reinterpret_cast<u32x4*>(&vrow[tl][d0 + e]) =
            *reinterpret_cast<const u32x4*>(v_new + src + e);
    }
    __syncthreads();
    uint16_t* vtile = v_cache + (base / kBlock * num_kv_heads + g) * (int64_t)(D * kBlock);
#pragma unroll
    for (int r = threadIdx.x; r < 2 * D; r += 256) {
      const int d = r >> 1, h = r & 1;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)vrow[8 * h + 2 * e][d] | ((uint32_t)vrow[8 * h + 2 * e + 1][d] << 16);
      *reinterpret_cast<u32x4*>(vtile + d * kBlock + 8 * h) = w;
    }
    return;
  }
  // V, any other slot pattern: element d goes to ((tile*D + d)*16 + off).
  uint16_t* vdst = v_cache + (tile * D + d0) * kBlock + off;
#pragma unroll
  for (int e = 0; e < EPT; e += 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(v_new + src + e);
    vdst[e * kBlock] = (uint16_t)(w & 0xFFFFu);
    vdst[(e + 1) * kBlock] = (uint16_t)(w >> 16);
  }
}

int launch_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                    void* k_cache, void* v_cache, int num_tokens, int num_kv_heads,
                    int head_dim, int64_t num_blocks, hipStream_t stream) {
  dim3 grid((num_tokens + 15) / 16, num_kv_heads);
  dim3 block(256);
  const int64_t num_slots = num_blocks * kBlock;
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, slot_mapping, (uint16_t*)k_cache,
                       (uint16_t*)v_cache, num_tokens, num_kv_heads, num_slots);
  };
  switch (head_dim) {
    case 64: args(write_kv_kernel<64>); break;
    case 128: args(write_kv_kernel<128>); break;
    case 256: args(write_kv_kernel<256>); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pa
