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
// column tiles).  The workgroup walks the keys 0..P_s+i_max in tiles of BK
// keys: the tile's blocks are looked up in the block table and copied
// (16-byte loads, next tile prefetched into registers) into LDS, K as
// [key][d] rows and V as [d][key] rows.  Waves then run, per 32-key pair:
//   S^T[key][col]  = K[key][:]   . Q^T[:][col]    (v_mfma_f32_16x16x32_bf16)
//   online softmax per column (base-2, scale*log2(e) folded in)
//   O^T[d][col]   += V^T[d][key] . P^T[key][col]
// with the same key permutation as the decode kernel: score-tile row r of
// the pair's two tiles holds key 8*(r/4) + r%4 (+4 for the second tile), so
// lane group c ends up with keys 8c..8c+7 of the pair -- exactly one 16-byte
// LDS read of a V^T row -- and P stays in registers as the B operand.
// Each K/V fragment read from LDS feeds NT MFMAs.
//
// Scheduling: workgroup slots with the most keys (last columns of a
// sequence) are dispatched first.
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr float kLog2e = 1.44269504088896341f;

template <int D, int NT, int BK, int NW>
struct PrefillCfg {
  static constexpr int kColsWave = 16 * NT;
  static constexpr int kCols = kColsWave * NW;
  static constexpr int kThreads = NW * 64;
  static constexpr int kKRow = D + 8;    // LDS K row stride (elements): 16-byte pad
  static constexpr int kVRow = BK + 8;   // LDS V^T row stride (elements)
  static constexpr int kBlocks = BK / kBlock;
  // 16-byte chunks per tile for K (and for V): kBlocks * 16 * D / 8.
  static constexpr int kChunks = kBlocks * 2 * D;
  static constexpr int kChunksPerThread = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "tile must split evenly over threads");
  static_assert(BK % 32 == 0, "tile is a whole number of 32-key pairs");
};

template <int D, int NT, int BK, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ prefix_lens, int num_seqs, int total_q, int max_q_len,
    int num_q_heads, int num_kv_heads, int group, int64_t num_blocks, int max_blocks,
    int nslots, float scale_log2) {
  using Cfg = PrefillCfg<D, NT, BK, NW>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int KROW = Cfg::kKRow;
  constexpr int VROW = Cfg::kVRow;
  constexpr int CPT = Cfg::kChunksPerThread;
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][BK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][D * VROW];

  const int per_slot = num_seqs * num_kv_heads;
  const int bid = blockIdx.x;
  const int slot = nslots - 1 - bid / per_slot;
  const int s = (bid % per_slot) / num_kv_heads;
  const int g = bid % num_kv_heads;

  const int q0 = cu_seqlens[s];
  const int q1 = cu_seqlens[s + 1];
  if (q0 < 0 || q1 > total_q || q1 <= q0) return;
  const int nq = min(q1 - q0, max_q_len);
  const int ncols = nq * group;
  const int c0 = slot * Cfg::kCols;
  if (c0 >= ncols) return;
  const int P = prefix_lens != nullptr ? prefix_lens[s] : 0;
  const int64_t L = (int64_t)P + (q1 - q0);
  const bool bad = P < 0 || (L + kBlock - 1) / kBlock > max_blocks;
  const int pos_max = (min(ncols, c0 + Cfg::kCols) - 1) / group;
  const int kend = bad ? 0 : P + pos_max + 1;  // keys this workgroup needs
  const int ntiles = (kend + BK - 1) / BK;
  const int32_t* bt = block_tables + (int64_t)s * max_blocks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int c = lane >> 4;

  // Columns of this lane: one per column tile.
  int lim[NT];       // last visible key, -1 for a column past the sequence
  int qrow[NT], qhead[NT];
  u32x4 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int cidx = c0 + wave * Cfg::kColsWave + 16 * nt + col;
    const bool ok = cidx < ncols;
    const int pos = ok ? cidx / group : 0;
    const int h = ok ? cidx - pos * group : 0;
    lim[nt] = ok ? P + pos : -1;
    qrow[nt] = q0 + pos;
    qhead[nt] = g * group + h;
    const uint16_t* qb = q + ((int64_t)qrow[nt] * num_q_heads + qhead[nt]) * D + 8 * c;
#pragma unroll
    for (int i = 0; i < KS; ++i) qf[nt][i] = ok ? load16(qb + 32 * i) : u32x4{0, 0, 0, 0};
  }

  f32x4 acc[NT][DT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = f32x4{0, 0, 0, 0};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  // ---- tile staging: global -> registers -> LDS ---------------------------
  u32x4 rk[CPT], rv[CPT];
  bool bad_entry = false;
  auto fetch = [&](int tile) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int ch = tid + e * Cfg::kThreads;
      const int b = ch / (2 * D);          // block within the tile
      const int w = ch - b * (2 * D);      // 16-byte chunk within the block tile
      const int lblk = tile * Cfg::kBlocks + b;
      const int kpos0 = lblk * kBlock;
      rk[e] = u32x4{0, 0, 0, 0};
      rv[e] = u32x4{0, 0, 0, 0};
      if (kpos0 < kend) {
        const int64_t phys = bt[lblk];
        if (phys >= 0 && phys < num_blocks) {
          const int64_t tbase = (phys * num_kv_heads + g) * (int64_t)(kBlock * D);
          rk[e] = load16(k_cache + tbase + 8 * w);
          u32x4 v = load16(v_cache + tbase + 8 * w);
          // V^T chunk w holds keys 8*(w&1)..+8 of d row w/2; keys at or past
          // kend are never weighted but may hold NaN: zero them.
          const int key0 = kpos0 + 8 * (w & 1);
          if (key0 + 8 > kend) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const uint32_t keep = ((key0 + 2 * x < kend) ? 0x0000FFFFu : 0u) |
                                    ((key0 + 2 * x + 1 < kend) ? 0xFFFF0000u : 0u);
              v[x] &= keep;
            }
          }
          rv[e] = v;
        } else {
          bad_entry = true;
        }
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int ch = tid + e * Cfg::kThreads;
      const int b = ch / (2 * D);
      const int w = ch - b * (2 * D);
      // K chunk w: key w/(D/8), d 8*(w%(D/8)).
      const int key = w / (D / 8);
      const int dk = 8 * (w - key * (D / 8));
      *reinterpret_cast<u32x4*>(&sk[buf][(b * kBlock + key) * KROW + dk]) = rk[e];
      // V^T chunk w: d row w/2, keys 8*(w&1).
      const int dv = w >> 1;
      *reinterpret_cast<u32x4*>(&sv[buf][dv * VROW + b * kBlock + 8 * (w & 1)]) = rv[e];
    }
  };

  // K row of score tile t, pair kp, for this lane: key 8*(col/4) + col%4 + 4t.
  const int krow0 = 8 * (col >> 2) + (col & 3);

  if (ntiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) fetch(tile + 1);
    const uint16_t* skb = sk[buf];
    const uint16_t* svb = sv[buf];
    auto run_tile = [&](auto hilo_tag) {
      constexpr bool HILO = decltype(hilo_tag)::value;
#pragma unroll
      for (int kp = 0; kp < BK / 32; ++kp) {
        f32x4 s0[NT], s1[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          s0[nt] = f32x4{0, 0, 0, 0};
          s1[nt] = f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const u32x4 a0 =
              *reinterpret_cast<const u32x4*>(&skb[(32 * kp + krow0) * KROW + 32 * i + 8 * c]);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(
              &skb[(32 * kp + krow0 + 4) * KROW + 32 * i + 8 * c]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            s0[nt] = mfma16x16x32(a0, qf[nt][i], s0[nt]);
            s1[nt] = mfma16x16x32(a1, qf[nt][i], s1[nt]);
          }
        }
        // Lane group c holds keys key0 + 0..7 (0..3 from s0, 4..7 from s1).
        const int key0 = tile * BK + 32 * kp + 8 * c;
        u32x4 pb[NT], pl[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float sc[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            sc[t] = (key0 + t <= lim[nt]) ? s0[nt][t] * scale_log2 : -INFINITY;
            sc[t + 4] = (key0 + 4 + t <= lim[nt]) ? s1[nt][t] * scale_log2 : -INFINITY;
          }
          float mx = sc[0];
#pragma unroll
          for (int t = 1; t < 8; ++t) mx = fmaxf(mx, sc[t]);
          mx = wave_xor_max(mx, 16);
          mx = wave_xor_max(mx, 32);
          const float m_new = fmaxf(m_run[nt], mx);
          const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
          const float alpha = fast_exp2(m_run[nt] - m_use);
          float psum = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = fast_exp2(sc[2 * e] - m_use);
            const float b = fast_exp2(sc[2 * e + 1] - m_use);
            const uint32_t w = pack_bf16x2(a, b);
            pb[nt][e] = w;
            if (HILO) {
              pl[nt][e] = pack_bf16x2(a - bf16_bits_to_f32(w & 0xFFFFu),
                                      b - bf16_bits_to_f32(w >> 16));
              psum += a + b;
            } else {
              psum += bf16_bits_to_f32(w & 0xFFFFu) + bf16_bits_to_f32(w >> 16);
            }
          }
          l_run[nt] = l_run[nt] * alpha + psum;
          m_run[nt] = m_new;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[nt][dt] *= alpha;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4 a =
              *reinterpret_cast<const u32x4*>(&svb[(16 * dt + col) * VROW + 32 * kp + 8 * c]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt][dt] = mfma16x16x32(a, pb[nt], acc[nt][dt]);
            if (HILO) acc[nt][dt] = mfma16x16x32(a, pl[nt], acc[nt][dt]);
          }
        }
      }
    };
    // The first tile holds every key of the shortest causal rows, whose
    // outputs are averages of a few values: there P enters the matrix core
    // as a bf16 hi/lo pair so its rounding stays below the output rounding.
    if (tile == 0)
      run_tile(std::true_type{});
    else
      run_tile(std::false_type{});
    if (tile + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
  }

  const bool any_bad = __syncthreads_or(bad || bad_entry);
  const float nanv = __builtin_nanf("");
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = wave_xor_sum(l_run[nt], 16);
    l = wave_xor_sum(l, 32);
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

template <int D, int NT, int BK, int NW>
int launch_cfg(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* cu_seqlens,
               const int32_t* prefix_lens, int num_seqs, int total_q, int max_q_len,
               int num_q_heads, int num_kv_heads, int64_t num_blocks, int max_blocks_per_seq,
               float scale, hipStream_t stream) {
  using Cfg = PrefillCfg<D, NT, BK, NW>;
  const int group = num_q_heads / num_kv_heads;
  const int64_t cols = (int64_t)max_q_len * group;
  const int64_t nslots = (cols + Cfg::kCols - 1) / Cfg::kCols;
  const int64_t nwg = nslots * num_seqs * num_kv_heads;
  if (nwg > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL((prefill_kernel<D, NT, BK, NW>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                     stream, (uint16_t*)out, (const uint16_t*)q, (const uint16_t*)k_cache,
                     (const uint16_t*)v_cache, block_tables, cu_seqlens, prefix_lens, num_seqs,
                     total_q, max_q_len, num_q_heads, num_kv_heads, group, num_blocks,
                     max_blocks_per_seq, (int)nslots, scale * kLog2e);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

int launch_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* cu_seqlens,
                   const int32_t* prefix_lens, int num_seqs, int total_q, int max_q_len,
                   int num_q_heads, int num_kv_heads, int head_dim, int64_t num_blocks,
                   int max_blocks_per_seq, float scale, hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return launch_cfg<64, 4, 64, 4>(out, q, k_cache, v_cache, block_tables, cu_seqlens,
                                      prefix_lens, num_seqs, total_q, max_q_len, num_q_heads,
                                      num_kv_heads, num_blocks, max_blocks_per_seq, scale, stream);
    case 128:
      return launch_cfg<128, 2, 64, 4>(out, q, k_cache, v_cache, block_tables, cu_seqlens,
                                       prefix_lens, num_seqs, total_q, max_q_len, num_q_heads,
                                       num_kv_heads, num_blocks, max_blocks_per_seq, scale,
                                       stream);
    case 256:
      return launch_cfg<256, 2, 32, 4>(out, q, k_cache, v_cache, block_tables, cu_seqlens,
                                       prefix_lens, num_seqs, total_q, max_q_len, num_q_heads,
                                       num_kv_heads, num_blocks, max_blocks_per_seq, scale,
                                       stream);
    default:
      return -2;
  }
}

}  // namespace pa
