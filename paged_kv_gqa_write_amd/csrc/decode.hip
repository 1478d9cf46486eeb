// Paged GQA decode: split-K flash-decoding over block-tabled KV, plus the
// log-sum-exp reduce of the split-K pieces.  The same kernel serves decode
// with several query tokens per sequence (verifying a block of drafted
// tokens): every (query token, query head) pair of a KV head is one column.
//
// Work decomposition: one workgroup per (partition p, KV head g, sequence s,
// column chunk), NW waves per workgroup (3 or 4, chosen per shape in the
// launcher).  The partition's KV blocks are taken two at a time ("pairs", 32
// keys); wave w handles a contiguous range of pairs.  All G
// query heads of the KV head are processed together, so each K/V byte is read
// once.  A wave fetches the block-table entries of up to 32 pairs with one
// load (lane i holds entry i; pairs read them back with readlane) and keeps
// NBUF pairs of K/V loads in flight in a ring of register buffers.
//
// Both contractions run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16),
// with the columns -- (query token, query head) pairs, G heads per token --
// as the N dimension in NT tiles of 16 (padded when the count is not a
// multiple of 16); every tile reuses the pair's K/V registers:
//   S^T[key][head]  = K[key][:]   . Q^T[:][head]   (A = K rows, B = Q)
//   O^T[d][head]   += V^T[d][key] . P^T[key][head] (A = V^T rows, B = P)
// The score accumulator layout (lane l holds rows 4*(l/16)+r of column l%16)
// is chosen to be exactly the B-operand layout of the P.V product, so P never
// leaves registers: the 16 key rows of the two score tiles are a permutation
// of the pair's 32 keys such that lane group c ends up holding 8 consecutive
// keys of one block, which is also what one 16-byte load of a V^T row gives.
// K and V bytes go from HBM straight into MFMA operand registers with 16-byte
// loads.
//
// Softmax is online (running max m, running sum l per head, base-2
// exponentials with scale*log2(e) folded in); m is made uniform across the
// four lane groups of a head with two cross-lane max steps per pair, l is
// kept per lane and summed once at the end.  P enters the matrix core as a
// bf16 hi/lo pair (two products), which keeps its rounding error far below
// the bf16 output rounding; decode is memory-bound, so the extra products
// cost no time.  Waves are merged through LDS.
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr float kLn2 = 0.693147180559945309f;
constexpr int64_t kComputeUnits = 256;  // MI355X
constexpr float kLog2e = 1.44269504088896341f;

template <int D>
struct PairRegs {
  u32x4 k[2][D / 32];  // two score tiles x D/32 k-steps (A operand of S^T)
  u32x4 v[D / 16];     // D/16 d-tiles (A operand of O^T)
};

// Issue the loads of a pair (physical blocks x, y).  Every lane loads
// unconditionally from a valid block (a missing y block is replaced by x):
// keys past the partition's valid range are masked out of the scores and
// their V values are zeroed in compute_pair, so what such lanes read never
// matters, and straight-line loads keep the whole ring of pairs in flight.
template <int D>
__device__ __forceinline__ void load_pair(PairRegs<D>& r, const uint16_t* __restrict__ k_cache,
                                          const uint16_t* __restrict__ v_cache, int64_t physx,
                                          int64_t physy, int g, int hkv, int col, int c) {
  // K: score-tile row `col` -> key: group gr = col/4 picks the block (gr >= 2
  // -> second block) and the 4-key run 8*(gr&1) (+4 for the second tile).
  // The pool keeps each 32-wide slice i of the head dimension as the block's
  // 16 keys in 64-byte rows, so for k-step i a 4-key run is 256 contiguous
  // bytes and every load instruction covers whole 128-byte lines.
  {
    const int gr = col >> 2;
    const int key = 8 * (gr & 1) + (col & 3);
    const int64_t phys = gr >= 2 ? physy : physx;
    const uint16_t* base = k_cache + (phys * hkv + g) * kBlock * D + key * 32 + 8 * c;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
        r.k[t][i] = load16_stream(base + t * 4 * 32 + i * 32 * kBlock);
  }
  // V^T: lane group c reads keys 8*(c&1)..+8 of block (c >= 2 ? y : x), for
  // d row 16*dt + col.
  {
    const int64_t phys = c >= 2 ? physy : physx;
    const uint16_t* base = v_cache + ((phys * hkv + g) * D + col) * kBlock + 8 * (c & 1);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) r.v[dt] = load16_stream(base + dt * 16 * kBlock);
  }
}

// One pair of blocks for the NT column tiles.  Column (lane%16) of tile nt
// sees the keys below climit[nt] (its token's causal limit, at most `limit`,
// the end of the partition's valid keys).
template <int D, int NT>
__device__ __forceinline__ void compute_pair(PairRegs<D>& r, const u32x4 (&qf)[NT][D / 32],
                                             f32x4 (&acc)[NT][D / 16], float (&m_run)[NT],
                                             float (&l_run)[NT], int base_pos, int limit,
                                             const int (&climit)[NT], float scale_log2) {
  // Scores: tile 0 holds keys 8*(c&1)+0..3, tile 1 keys 8*(c&1)+4..7 of the
  // lane group's block.
  f32x4 s0[NT], s1[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    s0[nt] = f32x4{0, 0, 0, 0};
    s1[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      s0[nt] = mfma16x16x32(r.k[0][i], qf[nt][i], s0[nt]);
      s1[nt] = mfma16x16x32(r.k[1][i], qf[nt][i], s1[nt]);
    }
  }
  // P as a bf16 hi + lo pair: the two products together carry ~16 mantissa
  // bits of P, so rounding P costs nothing even when a few keys dominate.
  u32x4 pb_hi[NT], pb_lo[NT];
  float alpha[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float sc[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc[t] = (base_pos + t < climit[nt]) ? s0[nt][t] * scale_log2 : -INFINITY;
      sc[t + 4] = (base_pos + 4 + t < climit[nt]) ? s1[nt][t] * scale_log2 : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) mx = fmaxf(mx, sc[t]);
    if constexpr (D <= 128) {  // head_dim 256: the shuffle form measured faster
      mx = xor16_max(mx);
      mx = xor32_max(mx);
    } else {
      mx = wave_xor_max(mx, 16);
      mx = wave_xor_max(mx, 32);
    }
    const float m_new = fmaxf(m_run[nt], mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    alpha[nt] = fast_exp2(m_run[nt] - m_use);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = fast_exp2(sc[2 * e] - m_use);
      const float b = fast_exp2(sc[2 * e + 1] - m_use);
      const uint32_t hi = pack_bf16x2(a, b);
      pb_hi[nt][e] = hi;
      pb_lo[nt][e] =
          pack_bf16x2(a - bf16_bits_to_f32(hi & 0xFFFFu), b - bf16_bits_to_f32(hi >> 16));
      psum += a + b;
    }
    l_run[nt] = l_run[nt] * alpha[nt] + psum;
    m_run[nt] = m_new;
  }
  // Keys past the valid range may hold anything (NaN included); their P is 0
  // but 0*NaN is NaN, so zero their V values before the product.
  if (base_pos + 8 > limit) {
    u32x4 keep;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      keep[e] = ((base_pos + 2 * e < limit) ? 0x0000FFFFu : 0u) |
                ((base_pos + 2 * e + 1 < limit) ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) r.v[dt] &= keep;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      acc[nt][dt] *= alpha[nt];
      acc[nt][dt] = mfma16x16x32(r.v[dt], pb_hi[nt], acc[nt][dt]);
      acc[nt][dt] = mfma16x16x32(r.v[dt], pb_lo[nt], acc[nt][dt]);
    }
}

// Replaces, in a pair's loaded registers, the key at pair-relative position
// `rel` (0..31) by the new token's K row pieces `newk` and V values `newv`:
// the pool may not hold that token yet when the decode kernel appends it
// itself.  Lane (col, c) holds K rows 8*(gr&1) + (col&3) + 4t (+16 in the
// second block, gr = col/4) for tiles t = 0, 1, and V^T keys lane_key0..+7
// of d = 16*dt + col.
template <int D>
__device__ __forceinline__ void patch_pair(PairRegs<D>& r, const u32x4 (&newk)[D / 32],
                                           const uint32_t (&newv)[D / 16], int rel, int col,
                                           int lane_key0) {
  const int gr = col >> 2;
  const int krow = ((gr >= 2) ? kBlock : 0) + 8 * (gr & 1) + (col & 3);
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (krow + 4 * t == rel) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) r.k[t][i] = newk[i];
    }
  const int e = rel - lane_key0;
  if (e >= 0 && e < 8) {
    const int w = e >> 1;
    const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    const int sh = (e & 1) ? 16 : 0;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == w) r.v[dt][q] = (r.v[dt][q] & keep) | (newv[dt] << sh);
    }
  }
}

// Writes the appended token's K row pieces and V values, as lane (col, c)
// holds them (see patch_pair), into the pools at offset `off` of KV tile
// `tile` (= block * Hkv + KV head): lanes with col == 0 store the K pieces,
// lanes with c == 0 the V values.
template <int D>
__device__ __forceinline__ void store_new_row(uint16_t* k_pool, uint16_t* v_pool,
                                              const u32x4 (&newk)[D / 32],
                                              const uint32_t (&newv)[D / 16], int64_t tile,
                                              int off, int col, int c) {
  if (col == 0) {
    uint16_t* kd = k_pool + tile * kBlock * D + off * 32 + 8 * c;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) *reinterpret_cast<u32x4*>(kd + i * 32 * kBlock) = newk[i];
  }
  if (c == 0) {
    uint16_t* vd = v_pool + (tile * D + col) * kBlock + off;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vd[16 * dt * kBlock] = (uint16_t)newv[dt];
  }
}

// As patch_pair and store_new_row, with the new token's K and V rows read
// from this wave's LDS copy (kr, vr: D elements each) instead of registers.
template <int D>
__device__ __forceinline__ void patch_pair_lds(PairRegs<D>& r, const uint16_t* kr,
                                               const uint16_t* vr, int rel, int col, int c,
                                               int lane_key0) {
  const int gr = col >> 2;
  const int krow = ((gr >= 2) ? kBlock : 0) + 8 * (gr & 1) + (col & 3);
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (krow + 4 * t == rel) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) r.k[t][i] = *reinterpret_cast<const u32x4*>(kr + 8 * c + 32 * i);
    }
  const int e = rel - lane_key0;
  if (e >= 0 && e < 8) {
    const int w = e >> 1;
    const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    const int sh = (e & 1) ? 16 : 0;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const uint32_t nv = vr[16 * dt + col];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == w) r.v[dt][q] = (r.v[dt][q] & keep) | (nv << sh);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_new_row_lds(uint16_t* k_pool, uint16_t* v_pool,
                                                  const uint16_t* kr, const uint16_t* vr,
                                                  int64_t tile, int off, int col, int c) {
  if (col == 0) {
    uint16_t* kd = k_pool + tile * kBlock * D + off * 32 + 8 * c;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      *reinterpret_cast<u32x4*>(kd + i * 32 * kBlock) =
          *reinterpret_cast<const u32x4*>(kr + 8 * c + 32 * i);
  }
  if (c == 0) {
    uint16_t* vd = v_pool + (tile * D + col) * kBlock + off;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vd[16 * dt * kBlock] = vr[16 * dt + col];
  }
}

// Query tokens per sequence: query_len; columns per KV head: query_len *
// group, taken NT tiles of 16 at a time by `num_chunks` workgroups.  The
// chunks of one (partition, KV head, sequence) read the same K/V, so they
// are given launch indices that are equal modulo 8: the hardware deals
// workgroups to the 8 XCDs round-robin, so they run on one XCD and share
// its L2.
//
// APPEND (one query token per sequence): the kernel also appends the token's
// K/V (k_new/v_new [B, Hkv, D]) at position ctx-1 through the block table.
// The new row is loaded at the start; in the pair that covers position ctx-1
// the lanes take its values instead of the pool's (which may or may not have
// been written yet), and the wave that owns that pair writes
// the row into the pools.  k_pool/v_pool are the same pools as
// k_cache/v_cache; no reader depends on those stores.  The block number comes
// from the table entries the wave loads for its own pairs (a pair whose second
// block lies past the partition does not own a token in that block).  Position
// ctx-1 is the last key, so its pair is the last one the owning wave loads:
// the row is stored right behind that pair's loads, where no later wait of
// the wave depends on the store and its latency overlaps the pair's own (a
// store ahead of other pair loads delays them; one at the very end delays the
// launch's completion).  With two or more pairs in flight the row would not
// fit in registers beside the ring, so each wave copies it into its own LDS
// slot right after its first loads and reads it from there for the patch and
// the store.
//
// COMPACT (split launches of up to 64 sequences that need more than one
// dispatch round): items are ranked so that those holding keys come first
// and the empty ones (partitions past a sequence's length) last, so that
// every item with work is dispatched in the first round.  An empty
// workgroup still waits for its own small loads behind the batch's KV
// stream, and a live one dispatched after it would start that much later.
// Lane i loads sequence i's length; sequence s has n_s = min(ceil(ctx/ps),
// P) live partitions, and its live items come in the order (KV head,
// partition), as its empty ones do.  When every sequence fills every
// partition this is the plain order.
//
// Parameter order: the first eleven (14 dwords) are preloaded into SGPRs at
// wave launch; they are what the first loads need (table entries, context
// length, Q), so those loads do not wait for the kernel-argument fetch.
template <int D, int NW, int NBUF, int NT, bool APPEND, bool COMPACT>
__global__ __launch_bounds__(NW * 64, (APPEND && NBUF >= 2 && D <= 128) ? 2 : 1) void decode_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    const uint16_t* __restrict__ q, int num_partitions, int num_kv_heads, int max_blocks,
    int blocks_per_part, int num_chunks, int query_len, int group, int num_q_heads,
    uint16_t* __restrict__ out, float* __restrict__ part_out, float* __restrict__ part_lse,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* k_pool,
    uint16_t* v_pool, int num_seqs, int64_t num_blocks, float scale_log2) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  int item = blockIdx.x, chunk = 0;
  if (num_chunks > 1) {
    const int items = gridDim.x / num_chunks;
    const int base = (blockIdx.x / (8 * num_chunks)) * 8;
    const int width = min(8, items - base);
    const int r = blockIdx.x - base * num_chunks;
    chunk = r / width;
    item = base + r % width;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int col = lane & 15;
  const int c = lane >> 4;
  // Items are (sequence, KV head, partition), partition fastest.
  int p = item % num_partitions;
  int g = (item / num_partitions) % num_kv_heads;
  int s = item / (num_partitions * num_kv_heads);
  int cl = 0;  // COMPACT: lane i holds sequence i's length
  if constexpr (COMPACT) {
    cl = context_lens[min(lane, num_seqs - 1)];
    const int ps = blocks_per_part * kBlock;
    const int n = lane < num_seqs
                      ? (cl <= 0 ? 0 : (int)min((int64_t)num_partitions,
                                               ((int64_t)cl + ps - 1) / ps))
                      : 0;
    const int live = wave_total(n) * num_kv_heads;
    // Item `item` among the live items or among the empty ones.
    const bool in_live = item < live;
    const int per = in_live ? n : (lane < num_seqs ? num_partitions - n : 0);
    const int rr = in_live ? item : item - live;
    const int cnt = per * num_kv_heads;
    const int incl = wave_inclusive_scan(cnt);
    const uint64_t hit = __ballot(incl > rr);
    if (hit != 0) {  // always: the counts add up to the launch's items
      s = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
      const int off = rr - __builtin_amdgcn_readlane(incl - cnt, s);
      const int per1 = __builtin_amdgcn_readlane(per, s);  // > 0: s holds item rr
      g = off / per1;
      p = (in_live ? 0 : __builtin_amdgcn_readlane(n, s)) + off - g * per1;
    }
  }

  // Wave w takes the contiguous pair range [k0, k0+nk) of the partition.
  // The range comes from the partition size alone, so the block-table entries
  // can be fetched at the same time as the context length (it only trims the
  // range afterwards): the kernel starts with one round of independent loads.
  const int pb0 = p * blocks_per_part;
  const int full_pairs = (blocks_per_part + 1) / 2;
  const int k0 = (full_pairs * wave) / NW;
  const int wb0 = pb0 + 2 * k0;  // first block of this wave
  const int32_t* bt = block_tables + (int64_t)s * max_blocks;
  // Block-table entries of this wave's pairs, 32 pairs (64 entries) at a
  // time: lane i holds entry wb0 + 64*chunk + i; pair k reads lanes 2k, 2k+1.
  int ent = 0;
  auto load_entries = [&](int chunk) {
    const int b = wb0 + 64 * chunk + lane;
    ent = bt[min(b, max_blocks - 1)];
  };
  load_entries(0);

  const int ctx = COMPACT ? __builtin_amdgcn_readlane(cl, s) : context_lens[s];
  const int nblk = ctx > 0 ? (int)(((int64_t)ctx + kBlock - 1) / kBlock) : 0;
  bool bad = ctx < 0 || nblk > max_blocks ||
             (int64_t)ctx > (int64_t)num_partitions * blocks_per_part * kBlock ||
             (nblk > 0 && num_blocks <= 0) || (ctx > 0 && ctx < query_len);
  const int pb1 = bad ? pb0 : min(pb0 + blocks_per_part, nblk);
  const int limit = min(ctx, pb1 * kBlock);
  const int npairs = pb1 > pb0 ? (pb1 - pb0 + 1) / 2 : 0;
  const int k1 = min((full_pairs * (wave + 1)) / NW, npairs);
  const int nk = max(k1 - k0, 0);

  // Column j = (chunk*NT + nt)*16 + col is query token j / group, head
  // j % group of the KV head.  Token t sits at position ctx - query_len + t
  // and sees the keys below ctx - query_len + t + 1.  Columns past the last
  // token read token 0, head 0 instead: each column's softmax is independent
  // and those columns are never written, so their values do not matter.
  const int ncols = query_len * group;
  int crow[NT];    // output row (s*query_len + t)*Hq + head, or -1
  int climit[NT];  // keys visible to the column, within this partition
  u32x4 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int j = (chunk * NT + nt) * 16 + col;
    const bool live = j < ncols;
    const int t = live ? j / group : 0;
    const int hh = live ? j - t * group : 0;
    const int row = ((s * query_len + t) * num_q_heads) + g * group + hh;
    crow[nt] = live ? row : -1;
    climit[nt] = min(limit, ctx - query_len + t + 1);
    const uint16_t* qb = q + (int64_t)row * D + 8 * c;
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[nt][i] = load16(qb + 32 * i);
  }

  f32x4 acc[NT][DT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = f32x4{0, 0, 0, 0};
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  // Lane group c's keys start at block (c >= 2 ? y : x), offset 8*(c&1).
  const int lane_key0 = ((c >= 2) ? kBlock : 0) + 8 * (c & 1);

  // The appended token: in registers, this lane's pieces of its K row (the
  // d-slices its pool K loads cover) and its V values at d = 16*dt + col.
  const int pos_new = ctx - 1;
  // With two or more pairs in flight the row does not fit in registers next
  // to the ring: each wave keeps it in its own LDS slot instead.
  constexpr bool kRowLds = APPEND && NBUF >= 2;
  u32x4 newk[APPEND && !kRowLds ? KS : 1];
  uint32_t newv[APPEND && !kRowLds ? DT : 1];
  __shared__ __attribute__((aligned(16))) uint16_t sm_new[kRowLds ? NW : 1][2][D];
  constexpr int kRowWords = (D + 127) / 128;  // 2-element words per lane
  uint32_t nkw[kRowWords], nvw[kRowWords];
  if constexpr (kRowLds) {
    const int64_t src = ((int64_t)s * num_kv_heads + g) * D;
#pragma unroll
    for (int w = 0; w < kRowWords; ++w) {
      const int o = 2 * lane + 128 * w;
      if (o < D) {
        nkw[w] = *reinterpret_cast<const uint32_t*>(k_new + src + o);
        nvw[w] = *reinterpret_cast<const uint32_t*>(v_new + src + o);
      }
    }
  }
  if constexpr (APPEND && !kRowLds) {
    const int64_t src = ((int64_t)s * num_kv_heads + g) * D;
#pragma unroll
    for (int i = 0; i < KS; ++i) newk[i] = load16(k_new + src + 8 * c + 32 * i);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) newv[dt] = v_new[src + 16 * dt + col];
  }

  // Issue the loads of this wave's pair k into `r`.  An entry outside the
  // pool marks the sequence bad (NaN output) and is replaced by block 0 so
  // the loads stay in bounds (num_blocks == 0 never gets here: see above).
  int64_t pend_blk = -1;
  auto store_pending = [&]() {
    if constexpr (kRowLds) {
      if (pend_blk >= 0) {
        store_new_row_lds<D>(k_pool, v_pool, sm_new[wave][0], sm_new[wave][1],
                             pend_blk * num_kv_heads + g, pos_new % kBlock, col, c);
        pend_blk = -1;
      }
    }
  };
  auto issue = [&](int k, PairRegs<D>& r) {
    if ((k & 31) == 0 && k > 0) load_entries(k >> 5);
    const int e = 2 * (k & 31);
    int64_t px = __builtin_amdgcn_readlane(ent, e);
    int64_t py = __builtin_amdgcn_readlane(ent, e + 1);
    const bool hy = wb0 + 2 * k + 1 < pb1;
    const bool okx = px >= 0 && px < num_blocks;
    const bool oky = py >= 0 && py < num_blocks;
    bad |= !okx || (hy && !oky);
    int64_t store_blk = -1;
    if constexpr (APPEND) {
      const int rel = pos_new - (wb0 + 2 * k) * kBlock;  // wave-uniform
      if (rel >= 0 && rel < kBlock) store_blk = okx ? px : -1;
      else if (rel >= kBlock && rel < 2 * kBlock && hy) store_blk = oky ? py : -1;
    }
    px = okx ? px : 0;
    py = (hy && oky) ? py : px;
    load_pair<D>(r, k_cache, v_cache, px, py, g, num_kv_heads, col, c);
    // The pair holding position ctx-1 is the last one this wave loads: the
    // row goes out right behind its loads, so no wait of the wave follows it
    // (from LDS, right after the row is there when the pair is in the prologue).
    if constexpr (APPEND) {
      if (chunk == 0 && store_blk >= 0) {
        if constexpr (kRowLds)
          pend_blk = store_blk;
        else
          store_new_row<D>(k_pool, v_pool, newk, newv, store_blk * num_kv_heads + g,
                           pos_new % kBlock, col, c);
      }
    }
  };

  // Ring of NBUF register buffers: NBUF pairs are in flight while one is
  // consumed; buffer b always holds pairs b, b+NBUF, b+2*NBUF, ...
  PairRegs<D> buf[NBUF];
#pragma unroll
  for (int b = 0; b < NBUF; ++b)
    if (b < nk) issue(b, buf[b]);
  if constexpr (kRowLds) {
#pragma unroll
    for (int w = 0; w < kRowWords; ++w) {
      const int o = 2 * lane + 128 * w;
      if (o < D) {
        *reinterpret_cast<uint32_t*>(&sm_new[wave][0][o]) = nkw[w];
        *reinterpret_cast<uint32_t*>(&sm_new[wave][1][o]) = nvw[w];
      }
    }
    store_pending();
  }
  for (int kb = 0; kb < nk; kb += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int k = kb + b;
      if (k < nk) {
        if constexpr (APPEND) {
          const int rel = pos_new - (wb0 + 2 * k) * kBlock;  // wave-uniform
          if (rel >= 0 && rel < 2 * kBlock) {
            if constexpr (kRowLds)
              patch_pair_lds<D>(buf[b], sm_new[wave][0], sm_new[wave][1], rel, col, c, lane_key0);
            else
              patch_pair<D>(buf[b], newk, newv, rel, col, lane_key0);
          }
        }
        compute_pair<D, NT>(buf[b], qf, acc, m_run, l_run, (wb0 + 2 * k) * kBlock + lane_key0,
                            limit, climit, scale_log2);
        if (k + NBUF < nk) {
          issue(k + NBUF, buf[b]);
          store_pending();
        }
      }
    }
  }

  // Per-wave totals: l over the four lane groups of each column.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if constexpr (D <= 128) {
      l_run[nt] = xor16_sum(l_run[nt]);
      l_run[nt] = xor32_sum(l_run[nt]);
    } else {
      l_run[nt] = wave_xor_sum(l_run[nt], 16);
      l_run[nt] = wave_xor_sum(l_run[nt], 32);
    }
  }

  // Merge the NW waves: common max M per column; every wave hands its
  // rescaled accumulators to LDS, and wave w then sums and stores the d-tiles
  // w, w + NW, ... over all waves, adding in wave order from wave 0 (fixed
  // order: deterministic, and the same sums as one wave adding them all).
  // The bad flag travels with each wave's (m, l): one barrier for both.
  __shared__ float sm_m[NW][NT][16];
  __shared__ float sm_l[NW][NT][16];
  __shared__ int sm_bad[NW];
  __shared__ f32x4 sm_o[NW > 1 ? NW : 1][NT][DT][64];
  if (lane < 16) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      sm_m[wave][nt][col] = m_run[nt];
      sm_l[wave][nt][col] = l_run[nt];
    }
  }
  {
    const int wb = __ballot(bad) != 0 ? 1 : 0;
    if (lane == 0) sm_bad[wave] = wb;
  }
  __syncthreads();
  bool any_bad = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= sm_bad[w] != 0;
  float M[NT], L[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    M[nt] = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M[nt] = fmaxf(M[nt], sm_m[w][nt][col]);
    L[nt] = 0.f;
    float f = 0.f;
    if (M[nt] != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) L[nt] += sm_l[w][nt][col] * fast_exp2(sm_m[w][nt][col] - M[nt]);
      f = fast_exp2(m_run[nt] - M[nt]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nt][dt] *= f;
  }
  if (NW > 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) sm_o[wave][nt][dt][lane] = acc[nt][dt];
    __syncthreads();
  }
  // d-tile dt of column tile nt, summed over the waves.
  auto merged = [&](int nt, int dt) -> f32x4 {
    if constexpr (NW == 1) {
      return acc[nt][0 * dt];  // unreachable for NW == 1 (see the loops below)
    } else {
      f32x4 a = sm_o[0][nt][dt][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) a += sm_o[w][nt][dt][lane];
      return a;
    }
  };

  // Lane (col, c) holds column col of each tile, d = 16*dt + 4*c + r.
  const float nanv = __builtin_nanf("");
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (crow[nt] < 0) continue;
    const int64_t row = crow[nt];
    const float inv = L[nt] > 0.f ? 1.f / L[nt] : 0.f;
    if (num_partitions == 1) {
      uint16_t* dst = out + row * D + 4 * c;
      auto put = [&](int dt, f32x4 a) {
        f32x4 o = a * inv;
        if (any_bad) o = f32x4{nanv, nanv, nanv, nanv};
        u32x2 w;
        w[0] = pack_bf16x2(o[0], o[1]);
        w[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2*>(dst + 16 * dt) = w;
      };
      if constexpr (NW == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) put(dt, acc[nt][dt]);
      } else {
        for (int dt = wave; dt < DT; dt += NW) put(dt, merged(nt, dt));
      }
    } else {
      float* dst = part_out + (row * num_partitions + p) * D + 4 * c;
      auto put = [&](int dt, f32x4 a) {
        f32x4 o = a * inv;
        if (any_bad) o = f32x4{nanv, nanv, nanv, nanv};
        *reinterpret_cast<f32x4*>(dst + 16 * dt) = o;
      };
      if constexpr (NW == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) put(dt, acc[nt][dt]);
      } else {
        for (int dt = wave; dt < DT; dt += NW) put(dt, merged(nt, dt));
      }
      if (wave == 0 && c == 0) {
        float lse = L[nt] > 0.f ? (M[nt] + fast_log2(L[nt])) * kLn2 : -INFINITY;
        if (any_bad) lse = nanv;
        part_lse[row * num_partitions + p] = lse;
      }
    }
  }
}

// One wave per output row (sequence, query token, query head).  Lane p holds partition p's LSE (64
// partitions per chunk), so the max and the weights take one load; weights
// are broadcast with readlane and each lane accumulates its D/64 elements.
// The context length, the first chunk of LSEs and the first PF partitions'
// pieces are all loaded up front from in-bounds addresses (masked once the
// length is known), so the kernel waits for memory once, not three times.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ part_out,
    const float* __restrict__ part_lse, const int32_t* __restrict__ context_lens,
    int rows_per_seq, int partition_size, int num_partitions) {
  constexpr int EPT = D / 64;
  constexpr int PF = 16;
  const int64_t row = blockIdx.x;  // (s * query_len + t) * Hq + h
  const int s = (int)(row / rows_per_seq);
  const int lane = threadIdx.x;
  const float* lse = part_lse + row * num_partitions;
  const float* po = part_out + row * num_partitions * D + lane * EPT;
  const int ctx = context_lens != nullptr ? context_lens[s] : 0;
  const float lse0 = lse[min(lane, num_partitions - 1)];
  float pre[PF][EPT];
#pragma unroll
  for (int p = 0; p < PF; ++p)
#pragma unroll
    for (int e = 0; e < EPT; ++e) pre[p][e] = po[(int64_t)min(p, num_partitions - 1) * D + e];

  int np = num_partitions;
  if (context_lens != nullptr)
    np = ctx <= 0 ? 0 : (int)min((int64_t)num_partitions,
                                 ((int64_t)ctx + partition_size - 1) / partition_size);
  float M = -INFINITY;
  // A negative length is invalid device data: NaN, as the decode kernel
  // itself gives such a sequence when it writes the output directly.
  bool nan_seen = context_lens != nullptr && ctx < 0;
  for (int p0 = 0; p0 < np; p0 += 64) {
    const float v = (p0 + lane < np) ? (p0 == 0 ? lse0 : lse[p0 + lane]) : -INFINITY;
    nan_seen |= v != v;
    M = fmaxf(M, v);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = wave_xor_max(M, m);
  nan_seen = __any(nan_seen);

  float o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int p0 = 0; p0 < np; p0 += 64) {
      const float lv = p0 == 0 ? lse0 : lse[min(p0 + lane, num_partitions - 1)];
      const float w = (p0 + lane < np) ? fast_exp2((lv - M) * kLog2e) : 0.f;
      const int cnt = min(64, np - p0);
      int j = 0;
      if (p0 == 0) {
        // Pieces already in registers.
#pragma unroll
        for (int p = 0; p < PF; ++p) {
          if (p < cnt) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), p));
            L += wj;
#pragma unroll
            for (int e = 0; e < EPT; ++e) o[e] += wj * pre[p][e];
          }
        }
        j = min(PF, cnt);
      }
#pragma unroll 4
      for (; j < cnt; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        L += wj;
        const float* src = po + (int64_t)(p0 + j) * D;
#pragma unroll
        for (int e = 0; e < EPT; ++e) o[e] += wj * src[e];
      }
    }
  }
  uint16_t* dst = out + row * D + lane * EPT;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    float val = L > 0.f ? o[e] / L : 0.f;
    if (nan_seen) val = __builtin_nanf("");
    dst[e] = f32_to_bf16_bits(val);
  }
}

}  // namespace

int launch_decode(void* out, float* part_out, float* part_lse, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  const int32_t* context_lens, const void* k_new, const void* v_new,
                  int num_seqs, int query_len, int num_q_heads, int num_kv_heads, int head_dim,
                  int64_t num_blocks, int max_blocks_per_seq, int partition_size,
                  int num_partitions, float scale, hipStream_t stream) {
  const bool append = k_new != nullptr;
  if (append && query_len != 1) return -2;
  const int group = num_q_heads / num_kv_heads;
  const int tiles = (query_len * group + 15) / 16;
  // Up to two column tiles share a wave's K/V registers; more tiles are
  // spread over column chunks (separate workgroups on the same XCD).  Two
  // tiles per wave halve the K/V reads per column but double a wave's math
  // and its accumulators (one wave per SIMD); when even then the launch
  // would not give every compute unit a workgroup, one tile per workgroup
  // and twice the workgroups finish sooner.
  const int64_t items = (int64_t)num_partitions * num_kv_heads * num_seqs;
  const int nt = (tiles >= 2 && items * ((tiles + 1) / 2) >= kComputeUnits) ? 2 : 1;
  const int chunks = (tiles + nt - 1) / nt;
  const int64_t nwg = items * chunks;
  if (nwg > 0x7FFFFFFF) return -2;
  const float scale_log2 = scale * kLog2e;
  const int bpp = partition_size / kBlock;
  // Ranked launch order (COMPACT) when a split launch of up to 64 sequences
  // needs more than one workgroup per compute unit (the kernel ranks one
  // sequence per lane); otherwise the plain order.
  const bool compact = num_partitions > 1 && num_seqs <= 64 && nwg > kComputeUnits;
  auto go = [&](auto kern, int nw) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(nw * 64), 0, stream, block_tables,
                       context_lens, (const uint16_t*)q, num_partitions, num_kv_heads,
                       max_blocks_per_seq, bpp, chunks, query_len, group, num_q_heads,
                       (uint16_t*)out, part_out, part_lse, (const uint16_t*)k_cache,
                       (const uint16_t*)v_cache, (const uint16_t*)k_new, (const uint16_t*)v_new,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, num_seqs, num_blocks, scale_log2);
  };
  // Waves per workgroup (3 or 4) and pairs in flight per wave.  head_dim 128: 3 waves,
  // so that with partitions of 9 pairs (the batch-8 plans) every wave takes
  // exactly 3 pairs (two-tile form, Qwen3-4B verify batch 8: 13.8 -> 13.1 us,
  // 12.8 with 2 pairs in flight).  The plain form keeps 2 pairs in flight
  // per wave (Qwen3-4B batch 8: 11.4 -> 10.1 us against 4 waves with 1 pair
  // in flight); the appending form keeps 2 as well, its new row in LDS
  // (10.6 -> 10.35 us; with the row in registers 2 pairs need 288 registers,
  // one wave per SIMD).  Once partitions hold 32 pairs or more, both
  // single-tile forms take 4 waves (the appending one with 1 pair in flight,
  // its row in registers: 50.6 against 50.9 us): the tail imbalance is small
  // there and the extra wave's loads in flight pay (appending, Qwen3-32B
  // batch 64 at 36 pairs: 52.0 -> 51.2 us, batch 4 x 8192 at 32: 25.5 ->
  // 25.1; plain, batch 64: 49.8 -> 49.1, 16 x 8192 in 2 x 4096: 87.3 ->
  // 85.5).  The two forms split partitions alike, so they give bit-identical
  // results.  head_dim 256: 4 waves; the plain form keeps 2 pairs in flight,
  // the appending form 1 with its row in registers.  With 2, the appending
  // wave must wait for both pairs before it can copy its row into LDS, and
  // every wave of the launch then waits for the whole first burst (hybrid
  // batch 25.27 -> 24.93 us, 32 x 1024 18.07 -> 16.79, 64 x 512 29.56 ->
  // 28.57, 4 x 16384 27.14 -> 26.70; the plain form loses with 1: 24.71 ->
  // 26.25 on the hybrid batch).  Re-measured with the K pool in 32-wide
  // slices, hybrid batch: appending 21.98 (2 pairs) vs 21.16 (1), plain
  // 21.13 (2) vs 22.34 (1).
  auto pick = [&](auto compact_tag) {
    constexpr bool C = decltype(compact_tag)::value;
    switch (head_dim * 8 + nt * 2 + (append ? 1 : 0)) {
      case 64 * 8 + 2: go(decode_kernel<64, 4, 4, 1, false, C>, 4); return 0;
      case 64 * 8 + 4: go(decode_kernel<64, 4, 4, 2, false, C>, 4); return 0;
      case 64 * 8 + 3: go(decode_kernel<64, 4, 4, 1, true, C>, 4); return 0;
      case 128 * 8 + 2:
        // Partitions of 32+ pairs: a second pair in flight pays only when two
        // workgroups share a CU (batch 64: 49.31 -> 48.50 us); with one
        // workgroup per CU one pair was faster with token-row K (4 x 8192:
        // 25.04 -> 24.44 us) and is level with the sliced pool (24.06 vs
        // 24.10).
        if (bpp >= 64 && nwg <= kComputeUnits) go(decode_kernel<128, 4, 1, 1, false, C>, 4);
        else if (bpp >= 64) go(decode_kernel<128, 4, 2, 1, false, C>, 4);
        else go(decode_kernel<128, 3, 2, 1, false, C>, 3);
        return 0;
      case 128 * 8 + 4: go(decode_kernel<128, 3, 2, 2, false, C>, 3); return 0;
      case 128 * 8 + 3:
        // The same occupancy rule for the appending form (with the K pool in
        // 32-wide slices: batch 64 48.61 -> 48.39 us with 2 pairs, 4 x 8192
        // 24.10 -> 24.28).
        if (bpp >= 64 && nwg <= kComputeUnits) go(decode_kernel<128, 4, 1, 1, true, C>, 4);
        else if (bpp >= 64) go(decode_kernel<128, 4, 2, 1, true, C>, 4);
        else go(decode_kernel<128, 3, 2, 1, true, C>, 3);
        return 0;
      case 256 * 8 + 2: go(decode_kernel<256, 4, 2, 1, false, C>, 4); return 0;
      case 256 * 8 + 4: go(decode_kernel<256, 4, 1, 2, false, C>, 4); return 0;
      case 256 * 8 + 3: go(decode_kernel<256, 4, 1, 1, true, C>, 4); return 0;
      default: return -2;
    }
  };
  const int rc = compact ? pick(std::true_type{}) : pick(std::false_type{});
  if (rc != 0) return rc;
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_decode_reduce(void* out, const float* part_out, const float* part_lse,
                         const int32_t* context_lens, int num_seqs, int query_len,
                         int num_q_heads, int head_dim, int partition_size, int num_partitions,
                         hipStream_t stream) {
  const int rows_per_seq = query_len * num_q_heads;
  const int64_t rows = (int64_t)num_seqs * rows_per_seq;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(64), 0, stream, (uint16_t*)out, part_out,
                       part_lse, context_lens, rows_per_seq, partition_size, num_partitions);
  };
  switch (head_dim) {
    case 64: go(decode_reduce_kernel<64>); break;
    case 128: go(decode_reduce_kernel<128>); break;
    case 256: go(decode_reduce_kernel<256>); break;
    default: return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pa
