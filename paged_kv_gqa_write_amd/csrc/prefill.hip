// Varlen causal prefill over the paged KV cache, with cached prefixes.
//
// Columns.  For one sequence s and KV head g, every (new token i, query head
// h of the group) pair is a "column" c = i*G + h; all columns of a KV head
// read the same keys, so grouping query heads into the 16-wide MFMA N
// dimension shares every K/V byte across the whole group.  Column c sees
// keys 0..P_s+i (P_s = cached prefix length).
//
// Work decomposition.  A workgroup of NW waves owns COLS = NW*16*NT
// consecutive columns of one (s, g); wave w owns 16*NT of them (NT MFMA
// column tiles, Q held in registers).  The workgroup walks the keys
// 0..P_s+i_max in tiles of BK keys.
//
// Staging.  Each tile's blocks are looked up in the block table (scalar
// loads) and copied HBM -> LDS with global_load_lds_dwordx4 (16 bytes per
// lane, no registers involved), S tiles deep: while tile t is consumed,
// tiles t+1..t+S-1 are in flight.  Each wave waits for its own copies with an
// explicit vmcnt and one raw barrier per tile publishes the tile and frees
// the buffer the next copy goes to.  A direct copy writes 1 KiB of LDS per
// wave instruction in lane order, so the source chunk each lane fetches
// chooses the layout.  A 16-byte LDS read (ds_read_b128) is served 16 lanes
// at a time, and on gfx950 (64 banks of 4 bytes) the 16 lanes served
// together are four 4-lane quads of one 32-lane half whose quad indices
// (lane/4 % 8) have the same bit parity, e.g. lanes 0-3, 12-15, 20-23, 24-27
// (measured with the bank-conflict counter).  The layouts give each such
// group 16 different 16-byte bank slots:
//   K tile   [BK keys][D], row r chunk j stored at chunk j ^ kswz(r) (the
//            pool's 32-wide slices are put back together into rows)
//   V^T tile [BK/16 blocks][D rows][16 keys], as in the pool (one contiguous
//            HBM read per copy)
//
// Math per 32-key pair (v_mfma_f32_16x16x32_bf16):
//   S^T[key][col]  = K[key][:]   . Q^T[:][col]
//   online softmax per column (base-2, scale*log2(e) folded into one FMA
//   per element, lazy rescale, row sums on the matrix core)
//   O^T[d][col]   += V^T[d][key] . P^T[key][col]
// Score-tile row r of the pair's two tiles holds key 8*(r/4) + r%4 (+4 for
// the second tile), so lane group c ends up with keys 8c..8c+7 of the pair,
// which is one 16-byte read of a V^T row: P stays in registers as the B
// operand.  Each K/V fragment read from LDS feeds NT MFMAs.
//
// Scheduling: workgroup slots with the most keys (last columns of a
// sequence) are dispatched first.
#include <atomic>
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr float kLog2e = 1.44269504088896341f;
// Softmax reference modes (see softmax_pair in the kernel).
enum { kFirst = 0, kFixed = 1, kLazy = 2 };
// Lazy mode: reference-max slack (log2 units) before the accumulators are
// rescaled.
constexpr float kRescaleLog2 = 8.f;
// Columns seeing at least this many keys take plain bf16 weights in the
// first tile too (see run_pass).
constexpr int kHiLoMinKeys = 128;

typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;

template <int D, int NT, int BK, int NW, int S>
struct PrefillCfg {
  static constexpr int kColsWave = 16 * NT;
  static constexpr int kCols = kColsWave * NW;
  static constexpr int kBlocks = BK / kBlock;
  static constexpr int kKBytes = BK * D * 2;
  static constexpr int kVBytes = BK * D * 2;
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static constexpr int kDmaK = kKBytes / 1024;     // 1 KiB wave copies per K tile
  static constexpr int kDma = kStageBytes / 1024;  // ... per stage
  static constexpr int kDmaPerWave = kDma / NW;
  static_assert(kDmaK % NW == 0 && (kDma - kDmaK) % NW == 0,
                "stage copies must split evenly over waves");
  static_assert(BK % 32 == 0, "tile is a whole number of 32-key pairs");
  static_assert(S >= 2 && S <= 4, "2..4 stages");
};

// K-tile swizzle: chunk (16 bytes) j of row r is stored at j ^ kswz(r).  For a
// 16-lane operand read the lanes' rows are 8*(l/4) + l%4 (+ a multiple of 4),
// and kswz maps them to 16 distinct values (D >= 128: rows are whole multiples
// of the 256-byte bank line) or, with the row parity, to 16 distinct bank
// quads (D = 64: two rows per bank line).
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 64)
    return (((r >> 3) & 3) << 1) | ((r >> 1) & 1);
  else
    return (((r >> 3) & 3) << 2) | (r & 3);
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until this wave's LDS operations are complete.
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// The first eleven parameters (14 dwords) are preloaded into SGPRs at wave
// launch: the work-item search starts from them without waiting for the
// kernel-argument fetch.
template <int D, int NT, int BK, int NW, int S, int WPE>
__global__ __launch_bounds__(NW * 64, WPE) void prefill_kernel(
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ prefix_lens, int num_seqs, int total_q, int max_q_len,
    int num_kv_heads, int max_blocks, int nslots, int slot_shift, int fold,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int num_q_heads, int group, int64_t num_blocks, float scale_log2) {
  using Cfg = PrefillCfg<D, NT, BK, NW, S>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int KB = Cfg::kKBytes;
  constexpr int DPW = Cfg::kDmaPerWave;
  // One LDS object per stage: distinct objects let the compiler see that the
  // buffer being read is not one being filled by the copies still in flight.
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[Cfg::kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[Cfg::kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t smem2[S >= 3 ? Cfg::kStageBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t smem3[S >= 4 ? Cfg::kStageBytes : 16];
  auto stage = [&](auto st) __attribute__((always_inline)) -> uint8_t* {
    constexpr int I = decltype(st)::value;
    if constexpr (I == 0) return smem0;
    else if constexpr (I == 1) return smem1;
    else if constexpr (I == 2) return smem2;
    else return smem3;
  };

  const int per_slot = num_seqs * num_kv_heads;
  const int bid = blockIdx.x;
  const int g = bid % num_kv_heads;
  int slot, s, q0, q1, P;
  // Table entries of this wave's block in tiles 0 and 1, fetched with the
  // sequence lengths when the longest-first order is computed (-1: none).
  int pre0 = -1, pre1 = -1;
  bool have_pre = false;
  if (slot_shift >= 0) {
    // Longest-first order of the (sequence, slot) work items.  The hardware
    // hands out workgroups in launch order, each to the next free slot of
    // its XCD, so launching items in decreasing cost keeps the finish times
    // level (greedy list scheduling).  A slot's cost is its number of key
    // tiles, ceil((P + min(n, (slot+1)*T)) / BK) with T = 2^slot_shift
    // tokens per slot; it grows with the slot, so "how many slots of sequence s
    // cost at least c" has a closed form.  Lane j handles sequence j
    // (num_seqs <= 64); every wave finds item number bid / Hkv on its own by
    // a binary search over the cost threshold.
    //
    // The first `fold` positions are the workgroups that start at once (every
    // slot of every CU).  Positions p and p + fold/2 land on the same CU, so
    // that round is folded: position p takes rank p, position p + fold/2
    // takes rank fold-1-p.  Each CU then holds one long and one short item
    // instead of two long ones, and the longest items, which bound the
    // launch when one sequence dominates, get their CU to themselves soon.
    // Later positions follow the plain longest-first order.
    const int ln = threadIdx.x & 63;
    int ns = 0, pl = 0, la = 0, lb = 0, lp = 0, le0 = -1, le1 = -1;
    // This wave's block of a tile (the same formula as below).
    const int wblk = (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * (Cfg::kDmaK / NW) *
                      (1024 / (2 * D))) / kBlock;
    if (ln < num_seqs) {
      la = cu_seqlens[ln];
      lb = cu_seqlens[ln + 1];
      lp = prefix_lens != nullptr ? prefix_lens[ln] : 0;
      ns = (la >= 0 && lb <= total_q && lb > la) ? min(lb - la, max_q_len) : 0;
      pl = max(lp, 0);
      const int32_t* row = block_tables + (int64_t)ln * max_blocks;
      if (wblk < max_blocks) le0 = row[wblk];
      if (Cfg::kBlocks + wblk < max_blocks) le1 = row[Cfg::kBlocks + wblk];
    }
    const int nsl = (ns + (1 << slot_shift) - 1) >> slot_shift;
    auto count = [&](int c) {  // slots of this lane's sequence costing >= c
      const int x = (c - 1) * BK - pl;
      return x < 0 ? nsl : (x >= ns ? 0 : nsl - (x >> slot_shift));
    };
    const int items = wave_total(nsl);
    const int pos = bid / num_kv_heads;
    if (pos >= items) return;
    const int nf = min(fold, items), half = nf >> 1;
    const int r = (pos < half || pos >= nf) ? pos : nf - 1 - (pos - half);
    const int cmax = wave_max_nonneg(nsl > 0 ? (pl + ns + BK - 1) / BK : 0);
    int lo = 1, hi = cmax + 1;  // total(lo) > r >= total(hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (wave_total(count(mid)) > r) lo = mid;
      else hi = mid;
    }
    const int a_lo = count(lo), a_hi = count(lo + 1);
    const int idx = r - wave_total(a_hi);
    // items of cost exactly lo, scanned over the lanes (sequences)
    const int incl = wave_inclusive_scan(a_lo - a_hi);
    const int excl = incl - (a_lo - a_hi);
    const uint64_t hit = __ballot(idx >= excl && idx < incl);
    if (hit == 0) return;  // unreachable: exactly one lane holds item idx
    s = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
    slot = __builtin_amdgcn_readlane(nsl - a_lo + (idx - excl), s);
    // The sequence's bounds and prefix are already in lane s.
    q0 = __builtin_amdgcn_readlane(la, s);
    q1 = __builtin_amdgcn_readlane(lb, s);
    P = __builtin_amdgcn_readlane(lp, s);
    pre0 = __builtin_amdgcn_readlane(le0, s);
    pre1 = __builtin_amdgcn_readlane(le1, s);
    have_pre = true;
  } else {
    slot = nslots - 1 - bid / per_slot;
    s = (bid % per_slot) / num_kv_heads;
    q0 = cu_seqlens[s];
    q1 = cu_seqlens[s + 1];
    P = prefix_lens != nullptr ? prefix_lens[s] : 0;
  }

  if (q0 < 0 || q1 > total_q || q1 <= q0) return;
  const int nq = min(q1 - q0, max_q_len);
  const int ncols = nq * group;
  const int c0 = slot * Cfg::kCols;
  if (c0 >= ncols) return;
  const int64_t L = (int64_t)P + (q1 - q0);
  const bool bad = P < 0 || (L + kBlock - 1) / kBlock > max_blocks || num_blocks <= 0;
  const int pos_max = (min(ncols, c0 + Cfg::kCols) - 1) / group;
  const int kend = bad ? 0 : P + pos_max + 1;  // keys this workgroup needs
  const int ntiles = (kend + BK - 1) / BK;
  const const_i32_ptr btc = (const_i32_ptr)(block_tables + (int64_t)s * max_blocks);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 15;
  const int c = lane >> 4;

  // Columns of this lane: one per column tile.  A column past the sequence
  // reads a valid row (its results are never written) and has limit -1.
  int lim[NT];
  int qrow[NT], qhead[NT];
  u32x4 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int cidx = c0 + wave * Cfg::kColsWave + 16 * nt + col;
    const bool ok = cidx < ncols;
    const int cc = ok ? cidx : ncols - 1;
    const int pos = cc / group;
    const int h = cc - pos * group;
    lim[nt] = ok ? P + pos : -1;
    qrow[nt] = q0 + pos;
    qhead[nt] = g * group + h;
    const uint16_t* qb = q + ((int64_t)qrow[nt] * num_q_heads + qhead[nt]) * D + 8 * c;
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[nt][i] = load16(qb + 32 * i);
  }
  // Q is left in flight: the first tile's copies are issued behind it, and
  // the wait before the first tile (vector-memory operations complete in
  // order) covers both.

  // Smallest causal limit over the wave's columns that are written (columns
  // past the sequence take whatever the plain form gives; never stored).
  // Columns grow with the lane and the tile, and so do their limits: lane 0's
  // first column has the smallest, and it is written whenever any column of
  // the wave is.
  const int lim0 = __builtin_amdgcn_readfirstlane(lim[0]);
  const int wave_min_lim = lim0 < 0 ? 0x7FFFFFFF : lim0;
  // A pair takes the masked form when it crosses a causal limit of one of this
  // wave's columns or reaches past kend (pair0 + 31 > wave_min_lim or
  // pair0 + 32 > kend), i.e. from pair0 = pmask on.
  const int pmask = min(wave_min_lim - 31, kend - 32) + 1;
  // The last tile when it reaches past kend (its V^T tail is zeroed), else -1.
  const int tail_tile = ntiles * BK > kend ? ntiles - 1 : -1;

  f32x4 acc[NT][DT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = f32x4{0, 0, 0, 0};
  // Running max (log2 domain) and the running row sum.  The sum is kept by
  // the matrix core: ONES(16x32) . P^T gives every row the column sum of P,
  // so l_acc[nt][0] is the column's sum of the bf16 weights actually used.
  float m_run[NT];
  f32x4 l_acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_acc[nt] = f32x4{0, 0, 0, 0};
  }
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8

  // ---- tile copies: HBM -> LDS ---------------------------------------------
  // A wave's K copies and V copies of a tile all fall in one block of the
  // tile (checked below), so each wave needs one table entry per tile.
  constexpr int KPW = Cfg::kDmaK / NW;
  constexpr int VPW = (Cfg::kDma - Cfg::kDmaK) / NW;
  constexpr int kRowsPer = 1024 / (2 * D);  // K rows per 1 KiB copy
  constexpr int kVPerBlock = D / 32;        // 1 KiB V^T copies per block
  static_assert(KPW * kRowsPer <= kBlock && kBlock % (KPW * kRowsPer) == 0, "K copies of a wave share a block");
  static_assert(VPW <= kVPerBlock && kVPerBlock % VPW == 0, "V copies of a wave share a block");
  static_assert((KPW * kRowsPer) * kVPerBlock == kBlock * VPW, "K and V copies of a wave share the block");
  const int wave_blk = (wave * KPW * kRowsPer) / kBlock;
  bool bad_entry = false;
  // Table entry of this wave's block in `tile` (block 0 stands in for blocks
  // past the keys needed -- never weighted -- and for bad entries).
  // Entries are int32: the range check runs in 32 bits on the scalar unit
  // (a pool of more than 2^31 - 1 blocks holds every non-negative entry).
  // One unsigned compare: a negative entry reads as 2^31 or more.
  const uint32_t nb_lim = num_blocks > 0x7FFFFFFF ? 0x80000000u : (uint32_t)num_blocks;
  // The wave's block of a tile holds needed keys for tiles below tlim_w:
  // block tile*kBlocks + wave_blk starts below kend.
  const int nblk_need = (kend + kBlock - 1) / kBlock;
  const int tlim_w = nblk_need > wave_blk ? (nblk_need - wave_blk + Cfg::kBlocks - 1) / Cfg::kBlocks : 0;
  auto checked_entry = [&](int tile, auto load) __attribute__((always_inline)) -> int {
    if (tile >= tlim_w) return 0;
    const int p = (int)load(tile * Cfg::kBlocks + wave_blk);
    if ((uint32_t)p >= nb_lim) {
      bad_entry = true;
      return 0;
    }
    return p;
  };
  auto entry_of = [&](int tile) __attribute__((always_inline)) -> int {
    return checked_entry(tile, [&](int lb) -> int { return btc[lb]; });
  };
  // Tiles 0 and 1 from the prefetched entries where there are some.
  auto first_entry = [&](int tile) __attribute__((always_inline)) -> int {
    if (!have_pre) return entry_of(tile);
    return checked_entry(tile, [&](int) -> int { return tile == 0 ? pre0 : pre1; });
  };
  // Element offset of (block, KV head g): a 32 x 32 -> 64-bit product (the
  // launcher checks that a block of all KV heads spans fewer than 2^31 elements).
  const uint32_t blk_elems = (uint32_t)num_kv_heads * (uint32_t)(kBlock * D);
  const uint32_t g_elems = (uint32_t)g * (uint32_t)(kBlock * D);
  auto issue = [&](int phys, uint8_t* sb) __attribute__((always_inline)) {
    const uint64_t tile_base = (uint64_t)(uint32_t)phys * blk_elems + g_elems;
    const uint16_t* kt = uniform_ptr(k_cache + tile_base);
    const uint16_t* vt = uniform_ptr(v_cache + tile_base);
#pragma unroll
    for (int k = 0; k < KPW; ++k) {
      const int m = wave * KPW + k;
      const int r0 = m * kRowsPer;
      const int off = 16 * lane;
      const int r = r0 + off / (2 * D);
      const int j = ((off % (2 * D)) / 16) ^ kswz<D>(r);
      // Chunk j of key row r sits in the pool's 32-wide slice j/4, as the
      // (j%4)-th 16 bytes of that slice's 64-byte row r: one copy takes the
      // same kRowsPer rows of every slice, whole 128-byte lines.
      __builtin_amdgcn_global_load_lds(
          kt + (uint32_t)((j >> 2) * 32 * kBlock + (r & 15) * 32 + 8 * (j & 3)), sb + 1024 * m,
          16, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < VPW; ++k) {
      const int mv = wave * VPW + k;
      __builtin_amdgcn_global_load_lds(vt + (uint32_t)(512 * (mv % kVPerBlock) + 8 * lane),
                                       sb + KB + 1024 * mv, 16, 0, 0);
    }
  };

  // Zero, in this wave's V^T copies of `tile`, the values of keys at or past
  // kend (tails of the last live block and stand-in blocks).  Lane l of copy
  // mv holds row d = 32*(mv % (D/32)) + l/2, keys 8*(l%2)..+7 of block
  // mv / (D/32) of the tile.
  auto zero_v_tail = [&](int tile, uint8_t* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < VPW; ++k) {
      const int mv = wave * VPW + k;
      const int key = tile * BK + kBlock * (mv / kVPerBlock) + 8 * (lane & 1);
      u32x4* p = reinterpret_cast<u32x4*>(sb + KB + 1024 * mv + 16 * lane);
      u32x4 v = *p;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] &= ((key + 2 * e < kend) ? 0x0000FFFFu : 0u) | ((key + 2 * e + 1 < kend) ? 0xFFFF0000u : 0u);
      *p = v;
    }
  };

  // Per-lane byte offsets of the LDS operand reads inside a stage, fixed for
  // the whole kernel: every read below is a lane base plus an immediate.
  // K: score tile t of pair kp reads row r = 32*kp + krow0 + 4t, whose
  // swizzle kswz(r) does not depend on kp or t (they only touch bits 2 and
  // 5 up); chunk 4i+c of that row.
  // V^T: block 2*kp + c/2 of the pair, row d = 16*dt + col, half c%2 (keys
  // 8*(c%2)..+7 of the block).  Within a 16-lane read group, the lanes with
  // c%2 = 0 cover every row residue d%8 once and so do those with c%2 = 1,
  // in opposite halves: 16 different slots.
  const int krow0 = 8 * (col >> 2) + (col & 3);
  int koff[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i) koff[i] = krow0 * (2 * D) + 16 * ((4 * i + c) ^ kswz<D>(krow0));
  const int voff = KB + (c >> 1) * (D * 32) + col * 32 + 16 * (c & 1);

  // Softmax of one 32-key pair whose raw scores are s0/s1: the bf16 weights
  // P (and their rounding residue for HILO) as the B operand of P.V.
  //
  // Reference max.  Exponentials are taken against a per-column reference
  // m_run (log2 domain), in one of three modes:
  //   kFirst  tile 0: m_run := max of the column's visible scores in the tile
  //           (every written column sees key 0, so this is a real score).
  //   kFixed  later tiles: m_run stays fixed.  A later score above it gives
  //           P = 2^(z - m_run) > 1, which fp32 and bf16 represent with the
  //           same relative precision; the pass is exact as long as nothing
  //           overflows, which the kernel checks afterwards (row sums below
  //           2^64, outputs finite).  No max is taken, no rescaling happens.
  //   kLazy   the exact fallback when that check fails: m_run moves to the
  //           new max whenever a score exceeds it by more than 2^8, and the
  //           accumulators are rescaled then.
  // MASK selects the form for pairs that cross a causal limit of this wave's
  // columns or reach past the workgroup's last key; every other pair takes
  // the plain form, which carries no per-key compares or selects.
  auto softmax_pair = [&](int key0, f32x4 (&s0)[NT], f32x4 (&s1)[NT], u32x4 (&pb)[NT],
                          u32x4 (&pl)[NT], auto mode_tag, auto mask_tag, auto hilo_tag)
      __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool HILO = decltype(hilo_tag)::value;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float sr[8];  // raw scores <q, k>
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sr[t] = s0[nt][t];
        sr[t + 4] = s1[nt][t];
      }
      bool vis[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) vis[t] = !MASK || key0 + t <= lim[nt];
      if constexpr (MODE != kFixed) {
        // The scale is >= 0, so the max can be taken on raw scores.
        float mraw = vis[0] ? sr[0] : -INFINITY;
#pragma unroll
        for (int t = 1; t < 8; ++t) mraw = fmaxf(mraw, vis[t] ? sr[t] : -INFINITY);
        const float mx = (mraw == -INFINITY) ? -INFINITY : mraw * scale_log2;
        if constexpr (MODE == kFirst) {
          // Max over the column's four lane groups; a column that sees no key
          // (past the sequence, never written) takes 0.
          float mall = xor16_max(mx);
          mall = xor32_max(mall);
          m_run[nt] = (mall == -INFINITY) ? 0.f : mall;
        } else {
          // The test is per lane but the update is wave-uniform; the new max
          // is reduced over the column's four lane groups, so m_run stays
          // equal across them.
          if (__any(mx > m_run[nt] + kRescaleLog2)) {
            float mall = xor16_max(mx);
            mall = xor32_max(mall);
            const float m_new = fmaxf(m_run[nt], mall);
            const float alpha = fast_exp2(m_run[nt] - m_new);
            l_acc[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[nt][dt] *= alpha;
            m_run[nt] = m_new;
          }
        }
      }
      const float neg_m = -m_run[nt];
      float pv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        pv[t] = fast_exp2(fmaf(sr[t], scale_log2, neg_m));
        if (MASK) pv[t] = vis[t] ? pv[t] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = pack_bf16x2(pv[2 * e], pv[2 * e + 1]);
        pb[nt][e] = w;
        if (HILO)
          pl[nt][e] = pack_bf16x2(pv[2 * e] - bf16_bits_to_f32(w & 0xFFFFu),
                                  pv[2 * e + 1] - bf16_bits_to_f32(w >> 16));
      }
    }
  };

  // Row sums and O^T += V^T . P^T for one pair.  One form for every pair:
  // the V^T values of keys at or past kend are zeroed in LDS beforehand
  // (their P is 0, but 0*NaN would be NaN), so no mask is needed here and
  // each accumulator has a single use (the matrix core updates it in place).
  auto pv_pair = [&](const uint8_t* sb, int kp, const u32x4 (&pb)[NT], const u32x4 (&pl)[NT],
                     auto hilo_tag) __attribute__((always_inline)) {
    constexpr bool HILO = decltype(hilo_tag)::value;
    // Keep the V^T operand reads below the score products: hoisted above
    // them they would be live together with the K operands (> 128 VGPRs).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      l_acc[nt] = mfma16x16x32(ones, pb[nt], l_acc[nt]);
      if (HILO) l_acc[nt] = mfma16x16x32(ones, pl[nt], l_acc[nt]);
    }
    const uint8_t* vr = sb + voff + kp * (2 * D * 32);
    u32x4 a[DT];
    auto vread = [&](int dt) __attribute__((always_inline)) {
      a[dt] = *reinterpret_cast<const u32x4*>(vr + dt * (16 * 32));
    };
    // V^T reads in flight ahead of the products.  While a tile copy into LDS
    // is in flight (from the first pair's score products to the next tile),
    // the compiler waits for all outstanding LDS reads at each use of a read
    // result, so a deeper read-ahead makes those full waits rarer: ten ahead
    // at head_dim 256 (register room at two waves per SIMD), two elsewhere.
    constexpr int VA = D >= 256 ? 10 : 2;
#pragma unroll
    for (int i = 0; i < VA; ++i)
      if (i < DT) vread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt + VA < DT) vread(dt + VA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[nt][dt] = mfma16x16x32(a[dt], pb[nt], acc[nt][dt]);
        if (HILO) acc[nt][dt] = mfma16x16x32(a[dt], pl[nt], acc[nt][dt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // FIRST: this is tile 0, whose first pair sets the reference max; the
  // tile's other pairs and all later tiles run in the pass's mode.
  // after_qk runs once per tile, right after the last pair's score products
  // are issued: the next tile's copies start there, off the path from the
  // barrier to the first LDS reads, and late enough that the earlier pairs'
  // LDS reads keep counted waits (with a copy into LDS in flight the compiler
  // waits for every outstanding LDS read).
  auto run_tile = [&](int tile, const uint8_t* sb, auto first_tag, auto mode_tag, auto hilo_tag,
                      auto plain_tag, auto&& after_qk) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    constexpr bool PLAIN = decltype(plain_tag)::value;  // every pair of the tile is plain
#pragma unroll
    for (int kp = 0; kp < BK / 32; ++kp) {
      f32x4 s0[NT], s1[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s0[nt] = f32x4{0, 0, 0, 0};
        s1[nt] = f32x4{0, 0, 0, 0};
      }
      u32x4 ka[KS], kb[KS];
      auto kread = [&](int i) __attribute__((always_inline)) {
        const uint8_t* kr = sb + koff[i] + 32 * kp * (2 * D);
        ka[i] = *reinterpret_cast<const u32x4*>(kr);
        kb[i] = *reinterpret_cast<const u32x4*>(kr + 4 * (2 * D));
      };
      // K reads in flight ahead of the products: two steps at head_dim 256
      // (two waves per SIMD leave registers for it and little else to hide the
      // LDS latency), one at head_dim 64/128 (the 128-register cap).
      constexpr int KA = D >= 256 ? 2 : 1;
#pragma unroll
      for (int i = 0; i < KA; ++i) kread(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        if (i + KA < KS) kread(i + KA);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          s0[nt] = mfma16x16x32(ka[i], qf[nt][i], s0[nt]);
          s1[nt] = mfma16x16x32(kb[i], qf[nt][i], s1[nt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kp == BK / 32 - 1) after_qk();
      // Lane group c holds keys key0 + 0..7 (0..3 from s0, 4..7 from s1).
      const int pair0 = tile * BK + 32 * kp;
      const int key0 = pair0 + 8 * c;
      // Wave-uniform: does the pair cross a causal limit of one of this
      // wave's columns, or reach past the keys this workgroup needs?
      u32x4 pb[NT], pl[NT];
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PLAIN) {
        softmax_pair(key0, s0, s1, pb, pl, mode_tag, std::false_type{}, hilo_tag);
      } else if (FIRST && kp == 0) {
        softmax_pair(key0, s0, s1, pb, pl, std::integral_constant<int, kFirst>{}, std::true_type{},
                     hilo_tag);
      } else if (pair0 >= pmask) {
        softmax_pair(key0, s0, s1, pb, pl, mode_tag, std::true_type{}, hilo_tag);
      } else {
        softmax_pair(key0, s0, s1, pb, pl, mode_tag, std::false_type{}, hilo_tag);
      }
      pv_pair(sb, kp, pb, pl, hilo_tag);
    }
  };

  // ---- pipeline: S-1 tiles issued ahead, one barrier per tile ---------------
  // At the top of tile t, this wave has issued tiles up to min(t+S-2,
  // ntiles-1); waiting for all but the later ones' copies leaves tile t
  // complete for this wave, and the barrier makes it complete for all waves
  // and guarantees everyone finished tile t-1, whose buffer the copy of tile
  // t+S-1 then reuses.  The loop is unrolled by S so that every buffer index
  // is a compile-time constant: the compiler can then tell the buffer being
  // read from the buffers still being filled and inserts no wait of its own.
  // Table entries are fetched one tile ahead of their use.  One pass over all
  // tiles in the given softmax mode; on return no copy is in flight.
  auto run_pass = [&](auto mode_tag, bool prefetched) __attribute__((always_inline)) {
    if (0 < ntiles)
      issue(prefetched ? first_entry(0) : entry_of(0), stage(std::integral_constant<int, 0>{}));
    // Two stages: tile 1 goes out at once too (stage 1 is free until then),
    // so it has the whole of tile 0 to arrive; from tile 1 on, tile t issues
    // tile t+1.
    if constexpr (S == 2)
      if (1 < ntiles)
        issue(prefetched ? first_entry(1) : entry_of(1), stage(std::integral_constant<int, 1>{}));
    if constexpr (S >= 3)
      if (1 < ntiles) issue(entry_of(1), stage(std::integral_constant<int, 1>{}));
    if constexpr (S >= 4)
      if (2 < ntiles) issue(entry_of(2), stage(std::integral_constant<int, 2>{}));
    int next_phys = entry_of(S == 2 ? 2 : S - 1);
    auto step = [&](int t, auto stage_tag, auto first_tag, auto hilo_tag, auto plain_tag)
        __attribute__((always_inline)) {
      constexpr int ST = decltype(stage_tag)::value;
      const int ahead = min(S - 2, ntiles - 1 - t);  // tiles issued after t
      if constexpr (S >= 4) {
        if (ahead >= 2) wait_vm<2 * (KPW + VPW)>();
        else if (ahead == 1) wait_vm<KPW + VPW>();
        else wait_vm<0>();
      } else if constexpr (S == 3) {
        if (ahead >= 1) wait_vm<KPW + VPW>();
        else wait_vm<0>();
      } else {
        if (decltype(first_tag)::value && 1 < ntiles) wait_vm<KPW + VPW>();  // tile 1 may stay in flight
        else wait_vm<0>();
      }
      // Last tile: zero the V^T values of keys at or past kend in this wave's
      // own copies (complete after the wait above) before publishing them.
      if (!decltype(plain_tag)::value && t == tail_tile) {
        zero_v_tail(t, stage(std::integral_constant<int, ST>{}));
        wait_lds();
      }
      __builtin_amdgcn_s_barrier();
      run_tile(t, stage(std::integral_constant<int, ST>{}), first_tag, mode_tag, hilo_tag, plain_tag,
               [&]() __attribute__((always_inline)) {
                 if constexpr (S == 2) {
                   if (!decltype(first_tag)::value && t + 1 < ntiles) {
                     issue(next_phys, stage(std::integral_constant<int, (ST + 1) % 2>{}));
                     next_phys = entry_of(t + 2);
                   }
                 } else if (t + S - 1 < ntiles) {
                   issue(next_phys, stage(std::integral_constant<int, (ST + S - 1) % S>{}));
                   next_phys = entry_of(t + S);
                 }
               });
    };
    // The first tile holds every key of the shortest causal rows, whose
    // outputs are averages of a few values: there P enters the matrix core
    // as a bf16 hi/lo pair so its rounding stays below the output rounding.
    // A wave whose columns all see at least kHiLoMinKeys keys averages the
    // first tile's rounding like any later tile's and takes the plain form
    // (each branch passes the one barrier of the tile).  The first tile
    // also sets the reference max.  It is peeled off so that the loops below
    // carry neither the first-tile softmax nor the hi/lo products.
    using no = std::false_type;
    if (0 < ntiles) {
      if (wave_min_lim >= kHiLoMinKeys - 1)
        step(0, std::integral_constant<int, 0>{}, std::true_type{}, no{}, no{});
      else
        step(0, std::integral_constant<int, 0>{}, std::true_type{}, std::true_type{}, no{});
    }
    int t0 = 1;
    if constexpr (S == 2) {
      // Tiles below tplain hold only plain pairs for this wave (the last
      // pair of tile t starts at t*BK + BK - 32 < pmask): a loop without
      // the masked forms or the tail test.  Waves may leave it at different
      // tiles; every wave still passes one barrier per tile.
      const int xp = pmask - BK + 32;
      const int tplain = min(ntiles, xp > 0 ? (xp + BK - 1) / BK : 0);
      using yes = std::true_type;
      wait_lds();  // no scalar load left pending into the loop
      for (; t0 + 1 < tplain; t0 += 2) {
        step(t0, std::integral_constant<int, 1>{}, no{}, no{}, yes{});
        step(t0 + 1, std::integral_constant<int, 0>{}, no{}, no{}, yes{});
      }
    }
    wait_lds();
    for (; t0 < ntiles; t0 += S) {
      step(t0, std::integral_constant<int, 1 % S>{}, no{}, no{}, no{});
      if (t0 + 1 < ntiles) step(t0 + 1, std::integral_constant<int, 2 % S>{}, no{}, no{}, no{});
      if constexpr (S >= 3)
        if (t0 + 2 < ntiles) step(t0 + 2, std::integral_constant<int, 3 % S>{}, no{}, no{}, no{});
      if constexpr (S >= 4)
        if (t0 + 3 < ntiles) step(t0 + 3, std::integral_constant<int, 4 % S>{}, no{}, no{}, no{});
    }
  };

  run_pass(std::integral_constant<int, kFixed>{}, true);

  // The fixed-reference pass is exact unless a score rose more than 2^64
  // above its column's first-tile max (or something overflowed): then the
  // workgroup runs again with the lazily rescaled reference.
  bool redo = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (lim[nt] < 0) continue;
    redo |= !(l_acc[nt][0] < 0x1p64f);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) redo |= !(fabsf(acc[nt][dt][e]) < INFINITY);
  }
  // Both flags over the workgroup in one exchange: a ballot per wave, one LDS
  // word per wave, one barrier (which also ends every wave's reads of the
  // stage buffers before a re-run copies into them).
  __shared__ int sm_flags[NW];
  {
    const int f = (__ballot(bad || bad_entry) != 0 ? 1 : 0) | (__ballot(redo) != 0 ? 2 : 0);
    if (lane == 0) sm_flags[wave] = f;
  }
  __syncthreads();
  int flags = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) flags |= sm_flags[w];
  const bool any_bad = (flags & 1) != 0;
  if ((flags & 2) != 0 && !any_bad) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      l_acc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = f32x4{0, 0, 0, 0};
    }
    run_pass(std::integral_constant<int, kLazy>{}, false);
  }

  const float nanv = __builtin_nanf("");
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = l_acc[nt][0];
    if (lim[nt] < 0) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* dst = out + ((int64_t)qrow[nt] * num_q_heads + qhead[nt]) * D + 4 * c;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 o = acc[nt][dt] * inv;
      if (any_bad) o = f32x4{nanv, nanv, nanv, nanv};
      u32x2 w;
      w[0] = pack_bf16x2(o[0], o[1]);
      w[1] = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<u32x2*>(dst + 16 * dt) = w;
    }
  }
}

template <int D, int NT, int BK, int NW, int S, int WPE>
int launch_cfg(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* cu_seqlens,
               const int32_t* prefix_lens, int num_seqs, int total_q, int max_q_len,
               int num_q_heads, int num_kv_heads, int64_t num_blocks, int max_blocks_per_seq,
               float scale, hipStream_t stream) {
  using Cfg = PrefillCfg<D, NT, BK, NW, S>;
  const int group = num_q_heads / num_kv_heads;
  const int64_t cols = (int64_t)max_q_len * group;
  const int64_t nslots = (cols + Cfg::kCols - 1) / Cfg::kCols;
  const int64_t nwg = nslots * num_seqs * num_kv_heads;
  if (nwg > 0x7FFFFFFF) return -2;
  // Longest-first launch order needs whole tokens per slot (kCols / group,
  // then a power of two) and one lane per sequence; otherwise slots are
  // launched in decreasing slot order.
  int slot_shift = -1;
  if (Cfg::kCols % group == 0 && num_seqs <= 64) {
    slot_shift = 0;
    while ((1 << slot_shift) < Cfg::kCols / group) ++slot_shift;
  }
  // Workgroups resident at once on this device (CUs x workgroups per CU),
  // found once per device; in item positions (one position = Hkv workgroups).
  static std::atomic<int> resident[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -3;
  int res = resident[dev].load(std::memory_order_relaxed);
  if (res == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(prefill_kernel<D, NT, BK, NW, S, WPE>), NW * 64,
            0) != hipSuccess)
      return -3;
    res = max(cus * per_cu, 1);
    resident[dev].store(res, std::memory_order_relaxed);
  }
  const int fold = res / num_kv_heads;
  hipLaunchKernelGGL((prefill_kernel<D, NT, BK, NW, S, WPE>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                     stream, block_tables, cu_seqlens, prefix_lens, num_seqs, total_q, max_q_len,
                     num_kv_heads, max_blocks_per_seq, (int)nslots, slot_shift, fold,
                     (uint16_t*)out, (const uint16_t*)q, (const uint16_t*)k_cache,
                     (const uint16_t*)v_cache, num_q_heads, group, num_blocks, scale * kLog2e);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

int launch_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* cu_seqlens,
                   const int32_t* prefix_lens, int num_seqs, int total_q, int max_q_len,
                   int num_q_heads, int num_kv_heads, int head_dim, int64_t num_blocks,
                   int max_blocks_per_seq, float scale, hipStream_t stream) {
#define PA_PREFILL_ARGS                                                                     \
  out, q, k_cache, v_cache, block_tables, cu_seqlens, prefix_lens, num_seqs, total_q,       \
      max_q_len, num_q_heads, num_kv_heads, num_blocks, max_blocks_per_seq, scale, stream
  switch (head_dim) {
    case 64: return launch_cfg<64, 1, 64, 8, 2, 4>(PA_PREFILL_ARGS);
    case 128: return launch_cfg<128, 1, 64, 8, 2, 4>(PA_PREFILL_ARGS);
    case 256: return launch_cfg<256, 1, 32, 8, 2, 1>(PA_PREFILL_ARGS);
    default: return -2;
  }
#undef PA_PREFILL_ARGS
}

}  // namespace pa
