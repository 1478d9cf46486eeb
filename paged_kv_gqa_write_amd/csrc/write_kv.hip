// Slot-mapped KV append into the paged pools (bit copies).
//
// One workgroup handles 16 consecutive new tokens of one KV head.  Thread
// (i, j) = (tid % 16, tid / 16) owns token i and the j-th sixteenth of the
// head dimension.  For K it copies that contiguous piece of the token's row;
// for the transposed V pool it writes each element to its (d, offset) place.
// Lanes 0..15 of a store instruction are the 16 tokens, so when the tokens'
// slots are consecutive in one block (the usual prefill case) every V store
// instruction covers whole 32-byte rows of the block tile.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int num_tokens, int num_kv_heads, int64_t num_slots) {
  constexpr int EPT = D / 16;  // elements per thread: 4, 8 or 16
  const int i = threadIdx.x & 15;
  const int j = threadIdx.x >> 4;
  const int t = blockIdx.x * 16 + i;
  const int g = blockIdx.y;
  if (t >= num_tokens) return;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int d0 = j * EPT;

  const int64_t src = ((int64_t)t * num_kv_heads + g) * D + d0;
  const int64_t tile = (blk * num_kv_heads + g);

  // K: contiguous EPT*2 bytes.
  uint16_t* kdst = k_cache + (tile * kBlock + off) * D + d0;
  if constexpr (EPT == 4) {
    *reinterpret_cast<u32x2*>(kdst) = *reinterpret_cast<const u32x2*>(k_new + src);
  } else {
#pragma unroll
    for (int e = 0; e < EPT; e += 8)
      *reinterpret_cast<u32x4*>(kdst + e) = *reinterpret_cast<const u32x4*>(k_new + src + e);
  }

  // V: element d goes to ((tile*D + d)*16 + off).
  uint16_t vals[EPT];
  if constexpr (EPT == 4) {
    u32x2 w = *reinterpret_cast<const u32x2*>(v_new + src);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      vals[2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      vals[2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  } else {
#pragma unroll
    for (int c = 0; c < EPT; c += 8) {
      u32x4 w = *reinterpret_cast<const u32x4*>(v_new + src + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vals[c + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
        vals[c + 2 * e + 1] = (uint16_t)(w[e] >> 16);
      }
    }
  }
  uint16_t* vdst = v_cache + (tile * D + d0) * kBlock + off;
#pragma unroll
  for (int e = 0; e < EPT; ++e) vdst[e * kBlock] = vals[e];
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
