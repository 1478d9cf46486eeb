// Device-side helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;      // tokens per KV block
constexpr int kWave = 64;       // gfx9 wavefront

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies row l%16 of A and column l%16 of B, each as 8 values of
// the reduction dimension (lane group l/16 picks which 8); it receives
// D[4*(l/16) + r][l%16] in element r.  Any assignment of the reduction index
// to (lane group, element) works as long as A and B use the same one.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// fp32 -> bf16 bits, round to nearest even, NaN preserved (hardware convert).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 through the two-lane vector conversion.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Global loads that go straight to registers; `nontemporal` variants hint
// the caches that the streamed KV is not reused.
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}
__device__ __forceinline__ float wave_xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, kWave);
}

// v combined with lane l ^ 16 (rows of 16 lanes) or l ^ 32 (halves of the
// wave) on the vector ALU.  Swapping a register's rows (halves) with a copy of
// itself leaves each lane its own value and its partner's, in one order or the
// other; max and + are commutative, so the results equal the shuffle forms
// above, bit for bit, without a trip through the LDS crossbar.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Uniform (scalar) copy of a wave-uniform value.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Scalar copy of a wave-uniform pointer.  Besides placing it in SGPRs, the
// opaque readfirstlane keeps the compiler from re-associating per-lane
// offsets into it, so `uniform_ptr(p) + lane_offset` addresses memory as
// scalar base + 32-bit vector offset.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Sum, max and inclusive prefix sum over the 64 lanes of a wave with DPP row
// operations (a few cycles each, no LDS crossbar).  The values are >= 0, so
// 0 serves as the identity for lanes a row mask leaves out.  Sum and max
// leave the total in lane 63.
__device__ __forceinline__ int dpp(int v, int ctrl, int row_mask) {
  switch (ctrl) {  // the control is an immediate
    case 0xB1: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    case 0x4E: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    case 0x141: return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    case 0x140: return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
    case 0x111: return __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
    case 0x112: return __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
    case 0x114: return __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
    case 0x118: return __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
    case 0x142: return __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
    default: return __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  }
}
__device__ __forceinline__ int wave_total(int v) {
  v += dpp(v, 0xB1, 0xF);   // quad_perm [1,0,3,2]
  v += dpp(v, 0x4E, 0xF);   // quad_perm [2,3,0,1]
  v += dpp(v, 0x141, 0xF);  // row_half_mirror
  v += dpp(v, 0x140, 0xF);  // row_mirror: every lane holds its row's sum
  v += dpp(v, 0x142, 0xA);  // row_bcast15 into rows 1 and 3
  v += dpp(v, 0x143, 0xC);  // row_bcast31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, dpp(v, 0xB1, 0xF));
  v = max(v, dpp(v, 0x4E, 0xF));
  v = max(v, dpp(v, 0x141, 0xF));
  v = max(v, dpp(v, 0x140, 0xF));
  v = max(v, dpp(v, 0x142, 0xA));
  v = max(v, dpp(v, 0x143, 0xC));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp(v, 0x111, 0xF);  // row_shr:1
  v += dpp(v, 0x112, 0xF);  // row_shr:2
  v += dpp(v, 0x114, 0xF);  // row_shr:4
  v += dpp(v, 0x118, 0xF);  // row_shr:8: scan within each row of 16
  v += dpp(v, 0x142, 0xA);  // rows 1 and 3 add the previous row's total
  v += dpp(v, 0x143, 0xC);  // rows 2 and 3 add the total of rows 0-1
  return v;
}

}  // namespace pa
