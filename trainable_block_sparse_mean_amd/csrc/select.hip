// Block selection: group-summed block scores + top-k.
//
// Scores: skill page "Infllm V2 Dense Sparse Switchable Attention",
// Architecture Overview (Hardware Kernel: log-sum-exp-normalised scores
// summed over the heads of a group) and Step 2 (compressed_attention: softmax
// of the scaled query / compressed-key products).  Selection: Step 2,
// selected_attention (top-k per query position) at block granularity (news
// summary, Technical Mechanism).
//
// One workgroup = 8 consecutive query tokens of one KV head, one token per
// wave; two workgroups share a CU up to 2048 key blocks (one past that), so
// that one's top-k, a scalar loop on one wave per token, overlaps the other's
// score passes.  The compressed keys stream through an LDS ring of CH-block
// chunks by direct-to-LDS loads: 4 slots in pairs (while one pair is read the
// next is in flight, one barrier per pair) where two workgroups' score rows
// leave room for it, else 2 slots, one chunk at a time.  Every wave reads
// the same chunk, so each chunk comes from L2 once per workgroup and pass.  For a token, S = Q k_cmp^T on 16x16x32 bf16 MFMAs puts
// the 16 heads of the group in the rows and 16 compressed blocks in the
// columns: lane (column hl, row quad gq) holds heads 4*gq .. 4*gq+3 of block
// 16*tile + hl.
//   pass 1: each lane keeps, per head, a running max (moved only when a
//           score exceeds it by 2^8) and a sum of exp2 over its blocks; the 16
//           lanes of a row are merged at the end -> per-head log-sum-exp
//           (log2 units).
//   pass 2: p = exp2(z - lse) per head, the group score of a block is the sum
//           over the lane's 4 heads and the 4 row quads (permlane swaps); it
//           goes to LDS only, never to HBM.
// Heads beyond G (G < 16) have zero queries and an infinite log-sum-exp, so
// they add exactly 0.  The top-k is an exact radix select on the fp32 bit
// patterns (non-negative floats order like their bits); ties are then taken
// lowest index first and the kept indices compacted in ascending order by
// ballot.
#include <type_traits>

#include "attn_common.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kSelWaves = 16;           // waves of the decode selection (the prefill kernel takes WAVES)
constexpr int kSelSlots = 4;            // LDS ring: the pair of chunks being read + the next pair
constexpr int kSelRowBytes = kD * 2;    // one compressed block
constexpr size_t kSelLdsMax = 160 * 1024;
constexpr float kSelSlack = 8.f;         // log2 units a running max may lag

// floats per token row of block scores in LDS
__host__ __device__ constexpr int sel_stride(int NB) { return (NB + 3) & ~3; }

template <int CH, int WAVES, int SL = kSelSlots>
constexpr size_t select_lds(int NB) {
  return static_cast<size_t>(SL) * CH * kSelRowBytes + static_cast<size_t>(WAVES) * sel_stride(NB) * 4;
}
// Workgroups of 8 tokens (8 waves), two per CU up to 2048 blocks: up to 512
// blocks with a ring of 64-block chunk pairs, up to 1536 with one 64-block
// chunk at a time, up to 2048 with one 32-block chunk at a time, so that both
// workgroups' score rows fit; past 2048 blocks one workgroup per CU (32-block
// chunk pairs) takes up to 4064.
constexpr int kSelWideWaves = 8;
static_assert(select_lds<64, kSelWideWaves>(512) <= kSelLdsMax / 2, "two 8-token workgroups of 512 blocks fit");
static_assert(select_lds<64, kSelWideWaves, 2>(1536) <= kSelLdsMax / 2, "two 8-token workgroups of 1536 blocks fit");
static_assert(select_lds<32, kSelWideWaves, 2>(2048) <= kSelLdsMax / 2, "two 8-token workgroups of 2048 blocks fit");
static_assert(select_lds<32, kSelWideWaves>(kMaxSparseBlocks) <= kSelLdsMax, "8 score rows of 4064 blocks fit");

// (max, sum of exp2 relative to the max) of the lanes l and l ^ mask within
// a 16-lane DPP row; dpp = row_ror control.  Both partners compute the same
// commutative expression, so after the four steps all 16 lanes hold
// bit-identical results.
template <int DPP>
__device__ __forceinline__ void lse_merge_row(float& m, float& l) {
  const float mo = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), DPP, 0xf, 0xf, false));
  const float lo = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(l), DPP, 0xf, 0xf, false));
  const float mn = fmaxf(m, mo);
  l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + (mo == -INFINITY ? 0.f : lo * exp2f(mo - mn));
  m = mn;
}

// Maximum (MAX) or sum over the 16 lanes of a DPP row, by rotations of 8, 4,
// 2 and 1 lanes (dpp = row_ror control).  Called with the four rotations in
// that order, it leaves the result in every lane of the row, bit-identical:
// each step combines two values that the lanes involved already agree on,
// and both maximum and sum are commutative.
template <int DPP, bool MAX>
__device__ __forceinline__ float row_reduce(float x) {
  const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), DPP, 0xf, 0xf, false));
  return MAX ? fmaxf(x, o) : x + o;
}

// Radix search for the threshold of an exact top-kk over keys x[t] (slot t
// of lane l holds a key, 0 where empty: every real key has a bit set).  From
// the state (tt, bit, cnt): tt a prefix of the answer with bits above `bit`
// decided, cnt = #{x >= tt} >= kk, each round tries bit `bit` of tt, keeping
// it if at least kk keys are >= the candidate.  It stops when every bit is
// decided, when exactly kk keys are >= tt (those kk keys are then the
// selection), or, if stop_at > 0, as soon as cnt <= stop_at.  Returns true if
// the threshold is final.
template <int NS>
__device__ __forceinline__ bool radix_rounds(const uint32_t (&x)[NS], int kk, uint32_t& tt, int& bit, int& cnt,
                                             int stop_at) {
  for (; bit >= 0; --bit) {
    if (cnt == kk) return true;
    if (cnt <= stop_at) return false;
    const uint32_t cv = tt | (1u << bit);
    int c = 0;
#pragma unroll
    for (int t = 0; t < NS; ++t) c += __popcll(__ballot(x[t] >= cv));
    if (c >= kk) {
      tt = cv;
      cnt = c;
    }
  }
  return true;
}

// The keys > tt and the first (lowest-index) ties at tt: kk of them, written
// to out[0 .. kk) in ascending index order.  Slot t of lane l holds key x[t]
// of index idx_at(t) (indices ascending in (t, lane) order); valid_at(t) says
// whether the slot holds a candidate.
template <int NS, typename Valid, typename Idx>
__device__ __forceinline__ void emit_topk(const uint32_t (&x)[NS], Valid valid_at, Idx idx_at, uint32_t tt, int kk,
                                          int first, int32_t* out, float* out_s) {
  int n_gt = 0;
#pragma unroll
  for (int t = 0; t < NS; ++t) n_gt += __popcll(__ballot(valid_at(t) && x[t] > tt));
  const int need_eq = kk - n_gt;  // ties at tt, lowest indices first
  int eq_before = 0, n_out = 0;
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const bool gt = valid_at(t) && x[t] > tt;
    const bool eq = valid_at(t) && x[t] == tt;
    const uint64_t eqm = __ballot(eq);
    const bool sel = gt || (eq && eq_before + mask_rank(eqm) < need_eq);
    eq_before += __popcll(eqm);
    const uint64_t selm = __ballot(sel);
    const int pos = n_out + mask_rank(selm);
    if (sel && pos < kk) {
      out[pos] = first + idx_at(t);
      if (out_s) out_s[pos] = __uint_as_float(x[t]);
    }
    n_out += __popcll(selm);
  }
}

// Exact top-kk (kk = topk < nC) of the nC scores cand[0 .. nC), candidate c
// in slot c / 64 of lane c % 64 (NS >= ceil(nC / 64) slots per lane).  Keys
// are the fp32 bit patterns with the sign cleared: every key is below 2^31,
// also for NaN scores (which order above +inf), and non-negative floats order
// like their keys.  A bitwise radix search finds a threshold tt: the kk-th
// largest key, or any prefix of it at or below which exactly kk keys lie.
// The keys above tt and the first (lowest-index) ties at tt are kept, written
// to out[0 .. kk) in ascending index order (index = first + c).
// Two shortcuts leave the result unchanged.  The bits every candidate shares
// are taken into tt at once (a round at such a bit keeps it exactly when the
// keys have it).  And with NS >= 8, once at most 16 NS keys are >= tt (keys
// below tt can no longer be selected), those keys and their indices are
// compacted, in index order, into the start of cand (this wave's own row:
// nC > 32 NS), and the search goes on over NS / 4 slots per lane.
template <int NS>
__device__ __forceinline__ void topk_row(float* cand, int nC, int topk, int first, int32_t* out, float* out_s,
                                         int lane) {
  const int kk = topk;
  uint32_t x[NS];
  auto valid = [&](int t) { return t * 64 + lane < nC; };
  auto index = [&](int t) { return t * 64 + lane; };
#pragma unroll
  for (int t = 0; t < NS; ++t) x[t] = valid(t) ? __float_as_uint(cand[index(t)]) & 0x7fffffffu : 0u;
  uint32_t tt = 0;
  int bit = 30;
  int cnt = nC;
  if constexpr (NS >= 4) {
    uint32_t o = 0u, a = 0xffffffffu;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      o |= x[t];
      a &= valid(t) ? x[t] : 0xffffffffu;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      o |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(o), m, 64));
      a &= static_cast<uint32_t>(__shfl_xor(static_cast<int>(a), m, 64));
    }
    const uint32_t d = o ^ a;  // bits in which the candidates differ (keys < 2^31)
    if (d == 0u) {
      tt = a;
      bit = -1;
    } else {
      bit = 31 - __builtin_clz(d);
      tt = a & ~((2u << bit) - 1u);
    }
  }
  // The search state is the same in every lane; in scalar registers the
  // rounds below are a scalar loop (otherwise the compiler keeps it in vector
  // registers and runs the loop under an exec mask).
  tt = __builtin_amdgcn_readfirstlane(tt);
  bit = __builtin_amdgcn_readfirstlane(bit);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  if constexpr (NS >= 8) {
    constexpr int S2 = NS / 4;
    constexpr int cap = 64 * S2;
    if (!radix_rounds<NS>(x, kk, tt, bit, cnt, cap)) {
      // compact the cnt keys >= tt: keys into cand[0 .. cnt), indices after them
      uint32_t* ck = reinterpret_cast<uint32_t*>(cand);
      int* ci = reinterpret_cast<int*>(cand) + cap;
      int base = 0;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const bool keep = valid(t) && x[t] >= tt;
        const uint64_t km = __ballot(keep);
        if (keep) {
          const int pos = base + mask_rank(km);
          ck[pos] = x[t];
          ci[pos] = index(t);
        }
        base += __popcll(km);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave reads back what its lanes wrote
      uint32_t y[S2];
      int yi[S2];
      bool yv[S2];
#pragma unroll
      for (int s2 = 0; s2 < S2; ++s2) {
        const int e = s2 * 64 + lane;
        yv[s2] = e < cnt;
        y[s2] = yv[s2] ? ck[e] : 0u;
        yi[s2] = yv[s2] ? ci[e] : 0;
      }
      radix_rounds<S2>(y, kk, tt, bit, cnt, 0);
      emit_topk<S2>(y, [&](int t) { return yv[t]; }, [&](int t) { return yi[t]; }, tt, kk, first, out, out_s);
      return;
    }
  } else {
    radix_rounds<NS>(x, kk, tt, bit, cnt, 0);
  }
  emit_topk<NS>(x, valid, index, tt, kk, first, out, out_s);
}

// R = 1: exact log-sum-exp in pass 1.  R > 1: the approximate one of
// infv2_select_blocks_strided_lse - pass 1 scores only every R-th visible
// compressed block, each standing for the R blocks of its group (the last
// group for its visible count), so it streams 1/R of the compressed keys.
// WAVES: tokens per workgroup (16 or 8).  MINB: workgroups a CU holds at
// once (2 holds the registers of a wave to 128, so that two 8-wave
// workgroups share a CU and one's top-k overlaps the other's passes).  SL:
// chunk slots in the ring (4: pairs of chunks, one barrier per pair; 2: one
// chunk at a time, to fit two workgroups' score rows of up to 2048 blocks).
template <int CH, int R, int WAVES, int MINB = 1, int SL = kSelSlots>
__global__ __launch_bounds__(WAVES * 64, MINB) void select_blocks_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ kc,
                                                                       int32_t* __restrict__ blk_idx,
                                                                       float* __restrict__ blk_score,
                                                                       AttnShape s) {
  constexpr int kTiles = CH / 16;               // 16-block MFMA tiles per chunk
  constexpr int kSlotBytes = CH * kSelRowBytes;
  constexpr int kDmaWaves = CH / 4;             // each moves 4 rows (1 KB) of a chunk
  extern __shared__ __align__(16) unsigned char sel_smem[];
  const uint32_t ring = lds_addr(sel_smem);
  float* sig_all = reinterpret_cast<float*>(sel_smem + SL * kSlotBytes);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar) from here on
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15;   // MFMA column: block within the tile
  const int gq = lane >> 4;   // row quad: heads 4*gq .. 4*gq+3
  const int g = blockIdx.y % s.H_kv;
  const int b = blockIdx.y / s.H_kv;
  const int r0 = (gridDim.x - 1 - blockIdx.x) * WAVES;  // latest (heaviest) tokens first
  const int r = r0 + wave;    // this wave's token
  const int off = seq_keys(s, b) - s.S_q;  // query row r sits at key position off + r
  const bool active = r < s.S_q;
  const int nv = active ? (off + r + 1) / kBS : 0;  // fully visible blocks
  const int r_last = min(r0 + WAVES, s.S_q) - 1;
  const int nv_max = (off + r_last + 1) / kBS;      // largest nv of the workgroup
  const int nch = (nv_max + CH - 1) / CH;             // pass 2 chunks (every block)
  const int nch1 = ((nv_max + R - 1) / R + CH - 1) / CH;  // pass 1 chunks (every R-th block)
  float* sig = sig_all + wave * sel_stride(s.NB);
  const float sl2 = s.scale_log2;

  // A operands: Q of the token (lane row = head hl, k-slots = dims 8*gq + 32*ks);
  // rows of heads >= G are zero
  bf16x8 qa[4];
  {
    const bool ok = active && hl < s.G;
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q + r) * kD + gq * 8;
    u32x4 raw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) raw[ks] = ok ? load16(qrow + ks * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = settle(as_bf16x8(raw[ks]));
  }
  const uint16_t* kg = kc + static_cast<size_t>(b * s.H_kv + g) * s.NB * kD;

  // chunk loads: row group d < kDmaWaves of a chunk is rows 4d .. 4d+3;
  // lane (sub, slot) fetches 16-byte column slot ^ swz(row) of row 4d + sub
  // into that row's slot (rows past NB - 1 re-read row NB - 1; never used).
  // Wave d loads group d of every chunk, and with 16 groups (64-block chunks)
  // and 8 waves also group d + 8 (rows 32 further: the same swizzle).
  static_assert(kDmaWaves == WAVES || kDmaWaves == 2 * WAVES, "loader waves per chunk");
  const int dwave = wave % kDmaWaves;
  const int drow = 4 * dwave + (lane >> 4);
  const uint32_t dcol = static_cast<uint32_t>(((lane & 15) ^ swz(drow)) << 4);
  const int nit = nch1 + nch;  // pass 1 chunks, then pass 2 chunks
  auto stage = [&](int it) {
    if (it < nit) {
      const int j = min(it < nch1 ? R * (it * CH + drow) : (it - nch1) * CH + drow, s.NB - 1);
      dma16(kg, static_cast<uint32_t>(j) * kSelRowBytes + dcol,
            ring + (it % SL) * kSlotBytes + dwave * 1024);
      if constexpr (kDmaWaves == 2 * WAVES) {
        const int j2 = min(it < nch1 ? R * (it * CH + drow + 32) : (it - nch1) * CH + drow + 32, s.NB - 1);
        dma16(kg, static_cast<uint32_t>(j2) * kSelRowBytes + dcol,
              ring + (it % SL) * kSlotBytes + (dwave + WAVES) * 1024);
      }
    }
  };
  // B-operand read offsets (row = block within the tile, k-step ks)
  uint32_t boff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) boff[ks] = hl * kSelRowBytes + (((4 * ks + gq) ^ swz(hl)) << 4);

  float m[4], l[4], lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
    lse2[i] = INFINITY;
  }

  // NT tiles of S from `buf` starting at tile t0: acc[t][i] = z(head 4*gq + i, block)
  auto scores = [&](const unsigned char* buf, int t0, auto nt_c, floatx4* acc) {
    constexpr int NT = decltype(nt_c)::value;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = mfma_16x16x32(qa[ks], as_bf16x8(load16(buf + boff[ks] + (t0 + t) * 16 * kSelRowBytes)), acc[t]);
  };
  // pass 1 update over NT tiles; masked scores (-inf) add nothing.  The
  // running max m (log2 units) only moves when a score exceeds it by more
  // than kSelSlack (decided per wave), so most chunks need no rescaling (the
  // branch is marked unlikely, or the compiler computes the rescale on every
  // chunk); the sum stays below 2^8 per term.  Maxima are IEEE maximum
  // (v_maximum3), which needs no quieting of its inputs first.
  auto lse_update = [&](const floatx4* acc, auto nt_c) {
    constexpr int NT = decltype(nt_c)::value;
    float mx[4];
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx[i] = acc[0][i];
#pragma unroll
      for (int t = 1; t < NT; ++t) mx[i] = __builtin_elementwise_maximum(mx[i], acc[t][i]);
      mx[i] *= sl2;
      need |= mx[i] > m[i] + kSelSlack;
    }
    if (__builtin_expect(__ballot(need) != 0, 0)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mn = __builtin_elementwise_maximum(m[i], mx[i]);
        l[i] = mn == -INFINITY ? 0.f : l[i] * __builtin_amdgcn_exp2f(m[i] - mn);
        m[i] = mn;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mref = m[i] == -INFINITY ? 0.f : m[i];
#pragma unroll
      for (int t = 0; t < NT; ++t) l[i] += __builtin_amdgcn_exp2f(fmaf(acc[t][i], sl2, -mref));
    }
  };
  // pass 2: group score of this lane's block in a tile (all 64 lanes get the
  // column sum)
  auto lane_score = [&](const floatx4& acc) {  // this lane's 4 heads
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) p += __builtin_amdgcn_exp2f(fmaf(acc[i], sl2, -lse2[i]));
    return p;
  };
  auto group_score = [&](const floatx4& acc) { return sum_xor32(sum_xor16(lane_score(acc))); };
  // The group scores of a whole chunk: the row quads' partial sums of the
  // kTiles tiles are exchanged in a transpose (quad pairs first, then wave
  // halves), so that quad gq ends with tile gq % kTiles, summed in the same
  // order as group_score: (quad 0 + quad 1) + (quad 2 + quad 3).
  auto chunk_scores = [&](const floatx4* acc) {
    auto swap16 = [](float a, float b) {  // even rows: a's own and b's odd rows; odd rows: the rest
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
      return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    };
    if constexpr (kTiles == 4) {
      // rows gq = 0, 2 hold tile 0 (u) and tile 2 (w), rows 1, 3 tiles 1 and 3, each summed over a quad pair
      const float u = swap16(lane_score(acc[0]), lane_score(acc[1]));
      const float w = swap16(lane_score(acc[2]), lane_score(acc[3]));
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(w), false, false);
      return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
      static_assert(kTiles == 2, "chunks of 32 or 64 blocks");
      return sum_xor32(swap16(lane_score(acc[0]), lane_score(acc[1])));
    }
  };
  using AllTiles = std::integral_constant<int, kTiles>;
  using OneTile = std::integral_constant<int, 1>;

  // chunk `it` of the sequence (pass 1 chunks, then pass 2 chunks), read from
  // its ring slot
  auto chunk = [&](int it) {
    if (it == nch1) {
      // end of pass 1: merge the 16 lanes of each row (one head per register
      // i), maximum first, then the lanes' sums rescaled to it: one
      // exponential per head instead of two per merge step
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mm = m[i];
        mm = row_reduce<0x128, true>(mm);
        mm = row_reduce<0x124, true>(mm);
        mm = row_reduce<0x122, true>(mm);
        mm = row_reduce<0x121, true>(mm);
        float ll = m[i] == -INFINITY ? 0.f : l[i] * exp2f(m[i] - mm);
        ll = row_reduce<0x128, false>(ll);
        ll = row_reduce<0x124, false>(ll);
        ll = row_reduce<0x122, false>(ll);
        ll = row_reduce<0x121, false>(ll);
        lse2[i] = 4 * gq + i < s.G ? mm + log2f(ll) : INFINITY;
      }
    }
    const unsigned char* buf = sel_smem + (it % SL) * kSlotBytes;
    if (it < nch1) {
      // pass 1 over rows jc .. jc + CH - 1 of the sampled sequence: sampled
      // row x is block R * x, standing for blocks R*x .. R*x + R-1 that are
      // visible (weight w: log2(w) / sl2 added to its scores)
      const int jc = it * CH;
      if (!active || R * jc >= nv) return;
      if (R * (jc + CH) <= nv) {
        floatx4 acc[kTiles];
        scores(buf, 0, AllTiles{}, acc);
        if constexpr (R > 1) {
          const float wl = log2f(static_cast<float>(R)) / sl2;
#pragma unroll
          for (int t = 0; t < kTiles; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] += wl;
        }
        lse_update(acc, AllTiles{});
      } else {
        for (int t = 0; t < kTiles && R * (jc + 16 * t) < nv; ++t) {
          floatx4 acc[1];
          scores(buf, t, OneTile{}, acc);
          const int j = R * (jc + 16 * t + hl);
          const int w = min(R, nv - j);  // visible blocks the sample stands for (<= 0: none)
          const float wl = R > 1 && w > 0 ? log2f(static_cast<float>(w)) / sl2 : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[0][i] = w > 0 ? (R > 1 ? acc[0][i] + wl : acc[0][i]) : -INFINITY;
          lse_update(acc, OneTile{});
        }
      }
      return;
    }
    const int jc = (it - nch1) * CH;  // first block of the pass 2 chunk
    if (!active || jc >= nv) return;
    const bool full = jc + CH <= nv;
    {
      if (full) {
        floatx4 acc[kTiles];
        scores(buf, 0, AllTiles{}, acc);
        // row quad gq stores tile gq % kTiles (quads with the same tile store
        // the same value to the same address)
        sig[jc + 16 * (gq % kTiles) + hl] = chunk_scores(acc);
      } else {
        for (int t = 0; t < kTiles && jc + 16 * t < nv; ++t) {
          floatx4 acc[1];
          scores(buf, t, OneTile{}, acc);
          const float p = group_score(acc[0]);
          const int j = jc + 16 * t + hl;
          if (gq == 0 && j < nv) sig[j] = p;
        }
      }
    }
  };

  if constexpr (SL == 2) {  // one chunk at a time (two workgroups per CU cover the waits)
    stage(0);
    for (int it = 0; it < nit; ++it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // chunk it is in LDS; every wave is done with it - 1
      stage(it + 1);    // into the slot chunk it - 1 used
      chunk(it);
    }
  } else {  // pairs of chunks, one barrier per pair
    stage(0);
    stage(1);
    for (int it = 0; it < nit; it += 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // chunks it, it + 1 are in LDS; every wave is done with it - 2, it - 1
      stage(it + 2);    // into the slots chunks it - 2, it - 1 used
      stage(it + 3);
      chunk(it);
      if (it + 1 < nit) chunk(it + 1);
    }
  }

  if (!active || s.topk == 0) return;  // no barriers below

  // ---- top-k over the candidates n_init .. qb - n_local ---------------------
  const int qb = (off + r) / kBS;
  const int lo = s.n_init;
  const int hi = qb - s.n_local;
  const int nC = hi >= lo ? hi - lo + 1 : 0;
  int32_t* out = blk_idx + (static_cast<size_t>(b * s.H_kv + g) * s.S_q + r) * s.topk;
  float* out_s = blk_score ? blk_score + (static_cast<size_t>(b * s.H_kv + g) * s.S_q + r) * s.topk : nullptr;

  if (nC <= s.topk) {  // every candidate is kept
    for (int e = lane; e < s.topk; e += 64) {
      out[e] = e < nC ? lo + e : -1;
      if (out_s) out_s[e] = e < nC ? sig[lo + e] : 0.f;
    }
    return;
  }
  const int nIt = (nC + 63) / 64;  // candidate slots per lane (<= 32 up to 2048 blocks, <= 64 past)
  if (nIt <= 1) topk_row<1>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 2) topk_row<2>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 4) topk_row<4>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 8) topk_row<8>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 16) topk_row<16>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (MINB > 1 || nIt <= 32) topk_row<32>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if constexpr (MINB == 1) topk_row<64>(sig + lo, nC, s.topk, lo, out, out_s, lane);
}

// Exact top-kk of nC (<= 2 * 1024) candidates cand[0 .. nC) by all 16 waves
// of a workgroup, with the same result as topk_row: keys are the fp32 bit
// patterns with the sign cleared; the kk-th largest key T is found digit by
// digit (bits 30..23, 22..15, 14..7, 6..0) from a shared 256-bin histogram of
// the keys that match the digits found so far; the keys above T and the
// first (lowest-index) ties at T are written to out[0 .. kk) in ascending
// index order, their positions from workgroup-wide prefix counts.  Thread t
// holds candidates t and t + 1024.  wsp: 304 words of LDS (the histogram,
// the digits found and the number of ties still to take, the per-wave
// counts of a prefix count).  Every thread of the workgroup calls this.
__device__ __forceinline__ void block_topk(const float* cand, int nC, int kk, int first, int32_t* out,
                                           float* out_s, uint32_t* wsp, int wave, int lane) {
  constexpr int NT = kSelWaves * 64;
  uint32_t* hist = wsp;        // [256]
  uint32_t* ctl = wsp + 256;   // prefix, ties to take
  uint32_t* wcnt = wsp + 256 + 16;  // [2][16 waves]
  const int t = threadIdx.x;
  uint32_t x[2];
  bool v[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    v[u] = t + u * NT < nC;
    x[u] = v[u] ? __float_as_uint(cand[t + u * NT]) & 0x7fffffffu : 0u;
  }
  uint32_t pre = 0u;
  int need = kk;  // the answer is the need-th largest key with the digits found so far
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sh = r < 3 ? 23 - 8 * r : 0;
    const uint32_t dmask = r < 3 ? 0xffu : 0x7fu;
    const uint32_t hmask = ~((1u << (sh + (r < 3 ? 8 : 7))) - 1u);  // the digits above this one
    if (t < 256) hist[t] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (v[u] && (x[u] & hmask) == pre) atomicAdd(&hist[(x[u] >> sh) & dmask], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane: digits 4*lane .. 4*lane+3; c_i = keys with a digit >= 4*lane + i
      const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 4 * lane);
      const uint32_t s4 = h[0] + h[1] + h[2] + h[3];
      uint32_t suf = s4;  // sum over lanes >= this one
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = static_cast<uint32_t>(__shfl_down(static_cast<int>(suf), d, 64));
        if (lane + d < 64) suf += o;
      }
      const uint32_t c3 = suf - s4 + h[3], c2 = c3 + h[2], c1 = c2 + h[1], c0 = c1 + h[0];
      const uint32_t nd = static_cast<uint32_t>(need);
      // the largest digit D with at least `need` keys at or above it
      const int D = __popcll(__ballot(c0 >= nd)) + __popcll(__ballot(c1 >= nd)) + __popcll(__ballot(c2 >= nd)) +
                    __popcll(__ballot(c3 >= nd)) - 1;
      const int d1 = D + 1;  // keys with a larger digit: c_(d1 % 4) of lane d1 / 4 (none past the last digit)
      const uint32_t mine = (d1 & 3) == 0 ? c0 : (d1 & 3) == 1 ? c1 : (d1 & 3) == 2 ? c2 : c3;
      const uint32_t above = d1 < 256 ? static_cast<uint32_t>(__shfl(static_cast<int>(mine), d1 >> 2, 64)) : 0u;
      if (lane == 0) {
        ctl[0] = pre | (static_cast<uint32_t>(D) << sh);
        ctl[1] = nd - above;
      }
    }
    __syncthreads();
    pre = ctl[0];
    need = static_cast<int>(ctl[1]);
  }
  // positions in index order (candidates 0 .. 1023 by thread, then 1024 ..):
  // workgroup-wide exclusive prefix counts of a flag
  auto prefix = [&](bool f0, bool f1, int& r0, int& r1) {
    const uint64_t b0 = __ballot(f0), b1 = __ballot(f1);
    if (lane == 0) {
      wcnt[wave] = static_cast<uint32_t>(__popcll(b0));
      wcnt[kSelWaves + wave] = static_cast<uint32_t>(__popcll(b1));
    }
    __syncthreads();
    int p0 = 0, all0 = 0, p1 = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const int c0 = static_cast<int>(wcnt[w]), c1 = static_cast<int>(wcnt[kSelWaves + w]);
      all0 += c0;
      if (w < wave) {
        p0 += c0;
        p1 += c1;
      }
    }
    r0 = p0 + mask_rank(b0);
    r1 = all0 + p1 + mask_rank(b1);
    __syncthreads();  // the counts are free for the next prefix
  };
  bool eq[2], sel[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) eq[u] = v[u] && x[u] == pre;
  int e0, e1;
  prefix(eq[0], eq[1], e0, e1);
  sel[0] = (v[0] && x[0] > pre) || (eq[0] && e0 < need);
  sel[1] = (v[1] && x[1] > pre) || (eq[1] && e1 < need);
  int q0, q1;
  prefix(sel[0], sel[1], q0, q1);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pos = u == 0 ? q0 : q1;
    if (sel[u] && pos < kk) {
      out[pos] = first + t + u * NT;
      if (out_s) out_s[pos] = __uint_as_float(x[u]);
    }
  }
}

// One query per sequence (decode): the 16 waves of a workgroup share the
// token and split its visible compressed blocks, so the whole workgroup works
// on one selection.  Wave w scores the 16-block tiles [w*tpw, (w+1)*tpw), its
// compressed keys loaded straight into the B operands (each block is read by
// one wave only, so nothing is staged in LDS), and keeps the scores in
// registers: the two passes become one pass over the keys.  The exact
// per-head log-sum-exp is formed from each head's maximum over the workgroup
// and then the sum of exp2 relative to it, both reduced through LDS; each
// wave turns its own scores into group scores in LDS, and wave 0 takes the
// top-k as the token-per-wave kernel does.  Same lane layout as that kernel.
constexpr int kDecTiles = 8;  // tiles per wave: 16 waves x 8 x 16 blocks covers 2048 blocks
constexpr int kDecQBytes = 4 * 64 * 16;  // the query's A operands, in lane order
static_assert(2 * kSelWaves * kMaxG >= 256 + 16 + 2 * kSelWaves, "block_topk's words fit in pmax and psum");
// The selection of (batch, KV head) bgi's one query, for a workgroup of 16
// waves, with dec_smem its LDS (decode_select_lds bytes); the kk indices and
// scores go to out / out_s (device or LDS memory; out_s may be null).  Every
// thread calls it; it ends without a barrier (only wave 0 writes the result
// when a wave's search takes the top-k).
__device__ __forceinline__ void select_decode_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                   int32_t* out, float* out_s, const AttnShape& s, int bgi,
                                                   unsigned char* dec_smem) {
  unsigned char* qsh = dec_smem;                                     // the query's A operands: [4 k-steps][64 lanes] x 16 B
  float* pmax = reinterpret_cast<float*>(dec_smem + kDecQBytes);     // [16 waves][16 heads]
  float* psum = pmax + kSelWaves * kMaxG;                            // [16 waves][16 heads]
  float* sig = psum + kSelWaves * kMaxG;                             // [NB]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15, gq = lane >> 4;
  const int g = bgi % s.H_kv;
  const int b = bgi / s.H_kv;
  const int pos = seq_keys(s, b) - 1;      // the query is the last key
  const int nv = (pos + 1) / kBS;          // fully visible blocks
  const int ntile = (nv + 15) / 16;
  const int tpw = (ntile + kSelWaves - 1) / kSelWaves;   // <= kDecTiles (NB <= 2048)
  const int tw0 = wave * tpw;
  const float sl2 = s.scale_log2;

  const int tend = min(ntile, tw0 + tpw);  // this wave's tiles: [tw0, tend)
  const uint16_t* kg = kc + static_cast<size_t>(b * s.H_kv + g) * s.NB * kD;
  // B operands of tile tw0 + t: lane (block hl of the tile, dims 8*gq + 32*ks);
  // rows past nv - 1 read row nv - 1 (their scores are dropped)
  auto kload = [&](int t, u32x4 (&kr)[4]) {
    const uint16_t* krow = kg + static_cast<size_t>(min(16 * (tw0 + t) + hl, max(nv - 1, 0))) * kD + gq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kr[ks] = load16(krow + ks * 32);
  };
  // the first two tiles' keys are loaded first.  The query's A operands (lane:
  // head hl, dims 8*gq + 32*ks) are the same for every wave: wave 0 loads them
  // and passes them on through LDS in lane order, so the CU's memory path,
  // which bounds this phase, carries the query once rather than once per wave.
  u32x4 kra[4], krb[4];
  if (tw0 < tend) kload(0, kra);
  if (tw0 + 1 < tend) kload(1, krb);
  if (wave == 0) {
    const bool ok = hl < s.G;
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q) * kD + gq * 8;
    u32x4 raw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) raw[ks] = ok ? load16(qrow + ks * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<u32x4*>(qsh + (ks * 64 + lane) * 16) = raw[ks];
  }
  __syncthreads();
  bf16x8 qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qsh + (ks * 64 + lane) * 16));

  // scores of this wave's tiles (log2 units); blocks >= nv are -inf.  Tiles go
  // in pairs, the next pair's keys loaded under the current pair's products.
  floatx4 z[kDecTiles];
  auto score = [&](const u32x4 (&kr)[4], int t) {
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma_16x16x32(qa[ks], as_bf16x8(kr[ks]), acc);
    const int j = 16 * (tw0 + t) + hl;
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = j < nv ? acc[i] * sl2 : -INFINITY;
    return r;
  };
#pragma unroll
  for (int t = 0; t < kDecTiles; ++t) z[t] = floatx4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int t = 0; t < kDecTiles; t += 2) {
    if (tw0 + t < tend) {  // wave-uniform
      z[t] = score(kra, t);
      if (tw0 + t + 1 < tend) z[t + 1] = score(krb, t + 1);
      if (t + 2 < kDecTiles && tw0 + t + 2 < tend) kload(t + 2, kra);
      if (t + 3 < kDecTiles && tw0 + t + 3 < tend) kload(t + 3, krb);
    }
  }
  // The exact per-head log-sum-exp, maximum first: the lane's tiles, the 16
  // lanes of its row (which hold the head's other blocks), then the waves;
  // then the sums of exp2 relative to that maximum, reduced the same way
  // (lane 0 of a row writes its row's sum, waves added in order).  Every wave
  // forms the result from the 16 waves' values in LDS.
  float mx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mx[i] = -INFINITY;
#pragma unroll
    for (int t = 0; t < kDecTiles; ++t)
      if (t < tpw) mx[i] = fmaxf(mx[i], z[t][i]);  // tiles past tpw are -inf
    mx[i] = row_reduce<0x128, true>(mx[i]);
    mx[i] = row_reduce<0x124, true>(mx[i]);
    mx[i] = row_reduce<0x122, true>(mx[i]);
    mx[i] = row_reduce<0x121, true>(mx[i]);
    if (hl == 0) pmax[wave * kMaxG + 4 * gq + i] = mx[i];
  }
  __syncthreads();
  floatx4 hm = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(pmax + w * kMaxG + 4 * gq);
#pragma unroll
    for (int i = 0; i < 4; ++i) hm[i] = fmaxf(hm[i], a[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float sm = 0.f;
    if (hm[i] != -INFINITY) {
#pragma unroll
      for (int t = 0; t < kDecTiles; ++t)
        if (t < tpw) sm += __builtin_amdgcn_exp2f(z[t][i] - hm[i]);
    }
    sm = row_reduce<0x128, false>(sm);
    sm = row_reduce<0x124, false>(sm);
    sm = row_reduce<0x122, false>(sm);
    sm = row_reduce<0x121, false>(sm);
    if (hl == 0) psum[wave * kMaxG + 4 * gq + i] = sm;
  }
  __syncthreads();
  floatx4 hs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) hs += *reinterpret_cast<const floatx4*>(psum + w * kMaxG + 4 * gq);
  float lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // heads >= G add nothing
    lse2[i] = 4 * gq + i < s.G && hm[i] != -INFINITY ? hm[i] + log2f(hs[i]) : INFINITY;
  // group scores of this wave's blocks
#pragma unroll
  for (int t = 0; t < kDecTiles; ++t) {
    if (t < tpw && tw0 + t < ntile) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) p += __builtin_amdgcn_exp2f(z[t][i] - lse2[i]);
      p = sum_xor32(sum_xor16(p));
      const int j = 16 * (tw0 + t) + hl;
      if (gq == 0 && j < nv) sig[j] = p;
    }
  }
  __syncthreads();
  if (s.topk == 0) return;

  const int qb = pos / kBS;
  const int lo = s.n_init;
  const int hi = qb - s.n_local;
  const int nC = hi >= lo ? hi - lo + 1 : 0;
  if (nC <= s.topk) {
    if (wave == 0) {
      for (int e = lane; e < s.topk; e += 64) {
        out[e] = e < nC ? lo + e : -1;
        if (out_s) out_s[e] = e < nC ? sig[lo + e] : 0.f;
      }
    }
    return;
  }
  const int nIt = (nC + 63) / 64;
  if (nIt > 8) {
    // more than 512 candidates: the whole workgroup (pmax / psum are free
    // again).  At 16 sequences of 128k keys this took the kernel from 31.6
    // to 27.4 us; at 512 candidates one wave's radix search is faster.
    block_topk(sig + lo, nC, s.topk, lo, out, out_s, reinterpret_cast<uint32_t*>(pmax), wave, lane);
    return;
  }
  if (wave != 0) return;
  if (nIt <= 1) topk_row<1>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 2) topk_row<2>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 4) topk_row<4>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else topk_row<8>(sig + lo, nC, s.topk, lo, out, out_s, lane);
}

__host__ __device__ constexpr size_t decode_select_lds(int NB) {
  return kDecQBytes + (static_cast<size_t>(kSelWaves) * kMaxG * 2 + sel_stride(NB)) * sizeof(float);
}

__global__ __launch_bounds__(kSelWaves * 64) void select_decode_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ kc,
                                                                       int32_t* __restrict__ blk_idx,
                                                                       float* __restrict__ blk_score, AttnShape s) {
  extern __shared__ __align__(16) unsigned char dec_smem[];
  const size_t row = static_cast<size_t>(blockIdx.x) * s.S_q * s.topk;
  select_decode_body(q, kc, blk_idx + row, blk_score ? blk_score + row : nullptr, s, blockIdx.x, dec_smem);
}

// ---------------------------------------------------------------------------
// Decode selection and block-sparse attention in one launch (news summary,
// Performance Evaluation: the method also serves decoding).  Workgroup
// (bg, split) first selects the top-k blocks of (batch, KV head) bg exactly
// as select_decode_kernel does, into LDS: the nsplit workgroups of bg repeat
// that selection, each on its own CU, rather than wait for a separate launch
// on 32 CUs and read its result back.  Then it attends split `split` of the
// token's union of blocks, as the split-KV sparse kernel does (the same item
// code, list and partials), and split 0 also stores the selection for the
// caller.  LDS: the 4-stage ring, then the top-k (indices and scores); the
// selection's own scratch overlays the ring.
// ---------------------------------------------------------------------------
static_assert(decode_select_lds(kMaxDecodeSelectBlocks) <= static_cast<size_t>(kStages) * kStageBytes,
              "the selection's scratch fits in the ring");

template <bool PAGED>
__global__ __launch_bounds__(kSelWaves * 64, 1) void decode_select_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int32_t* __restrict__ blk_idx, float* __restrict__ blk_score,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part, AttnShape s) {
  extern __shared__ __align__(1024) unsigned char smem[];
  int32_t* tk = reinterpret_cast<int32_t*>(smem + static_cast<size_t>(kStages) * kStageBytes);  // [topk]
  float* ts = reinterpret_cast<float*>(tk + s.topk);                                            // [topk]

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15, gq = lane >> 4;
  const int bg_i = blockIdx.x;
  const int g = bg_i % s.H_kv;
  const int b = bg_i / s.H_kv;
  const int split = blockIdx.y;

  // ---- the selection, into LDS ----------------------------------------------
  if (s.topk > 0) select_decode_body(q, kc, tk, ts, s, bg_i, smem);
  __syncthreads();
  if (split == 0) {
    const size_t row = static_cast<size_t>(bg_i) * s.topk;  // one query row
    for (int e = threadIdx.x; e < s.topk; e += kSelWaves * 64) {
      blk_idx[row + e] = tk[e];
      if (blk_score) blk_score[row + e] = ts[e];
    }
  }

  // ---- this split's share of the token's blocks ------------------------------
  const int S_k = seq_keys(s, b);
  const int off = S_k - 1;  // the query is the last key
  const int qb = off / kBS;
  const uint16_t* kg = PAGED ? k : k + static_cast<size_t>(bg_i) * s.S_k * kD;
  const uint16_t* vg = PAGED ? v : v + static_cast<size_t>(bg_i) * s.S_k * kD;
  const BlockSrc<PAGED> src{kg, vg, s.block_table, s.NB, s.num_pages, s.H_kv, b, g, S_k};
  const float sl2 = s.scale_log2;
  SparseState st;  // wave 0 holds the token; the other waves only stream
  {
    const bool valid = wave == 0 && hl < s.G;
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q) * kD + gq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) st.qf[ks] = valid ? as_bf16x8(load16(qrow + ks * 32)) : bf16x8{};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
    st.lim = off;
  }
  // The token's attended blocks in ascending order, without a list: the
  // initial blocks 0 .. n_i-1, then the selection (ascending, distinct, all
  // in n_init .. qb - n_local, so apart from the forced blocks), then the
  // window blocks w0 .. qb (those not already initial blocks): the union the
  // separate attention call builds from the same indices, in the same order.
  const int n_i = min(s.n_init, qb + 1);
  const int w0 = max(s.n_init, qb - s.n_local + 1);
  const int n_w = max(0, qb - w0 + 1);
  const int nC = max(0, qb - s.n_local - s.n_init + 1);  // the selection's candidates
  const int n_t = min(s.topk, nC);                      // and its valid entries
  const int nblk = n_i + n_t + n_w;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) st.qf[ks] = settle(st.qf[ks]);
  const int e_lo = static_cast<int>(static_cast<long long>(split) * nblk / s.nsplit);
  const int e_hi = static_cast<int>(static_cast<long long>(split + 1) * nblk / s.nsplit);
  const SparseLane spl = sparse_lane(hl, gq);
  auto entry_at = [&](int e) -> uint32_t {  // block | wave 0's token as its one member
    if (e >= nblk) return 0u;
    const int j = e < n_i ? e : e < n_i + n_t ? tk[e - n_i] : w0 + (e - n_i - n_t);
    return static_cast<uint32_t>(j) | (1u << 16);
  };
  stream_pairs<kSelWaves, false, 8>(smem, src, e_lo, e_hi, entry_at, wave, lane,
                                    [&](const unsigned char* const* stg, const int* js, uint32_t cur0, uint32_t cur1) {
    const uint32_t bit = 1u << (16 + wave);  // only wave 0's token is a member
    attend_pair(st, spl, stg, js, (cur0 & bit) != 0u, (cur1 & bit) != 0u, lane, sl2);
  });

  const float l = sum_xor32(sum_xor16(st.l));
  if (wave != 0 || hl >= s.G) return;
  const int h = g * s.G + hl;
  const size_t row = static_cast<size_t>(b * s.H_q + h) * s.S_q;
  if (s.nsplit > 1) {  // unnormalised partial of this split, merged by the combine kernel
    float* pr = part + (static_cast<size_t>(split) * s.B * s.H_q * s.S_q + row) * kPartFloats;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<floatx4*>(pr + 16 * dt + 4 * gq) = st.o[dt];
    if (gq == 0) {
      pr[128] = st.m;
      pr[129] = l;
    }
    return;
  }
  const float inv = 1.f / l;
  uint16_t* orow = out + row * kD + 4 * gq;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<u32x2*>(orow + 16 * dt) = u32x2{pack_bf16x2(st.o[dt][0] * inv, st.o[dt][1] * inv),
                                                     pack_bf16x2(st.o[dt][2] * inv, st.o[dt][3] * inv)};
  if (lse && gq == 0) lse[row] = (st.m + log2f(l)) * kLn2;
}

hipError_t launch_decode_select_attn(const uint16_t* q, const uint16_t* k_cmp, const uint16_t* k, const uint16_t* v,
                                     int32_t* blk_idx, float* blk_score, uint16_t* out, float* lse,
                                     const AttnShape& s_in, void* workspace, hipStream_t stream) {
  if (s_in.B == 0) return hipSuccess;
  AttnShape s = s_in;
  s.nsplit = sparse_splits(s.B, s.H_kv, s.S_q, s.topk);
  float* part = s.nsplit > 1 ? static_cast<float*>(workspace) : nullptr;
  const size_t lds = static_cast<size_t>(kStages) * kStageBytes + static_cast<size_t>(s.topk) * 8;
  const dim3 grid(s.B * s.H_kv, s.nsplit);
  if (s.block_table)
    hipLaunchKernelGGL(decode_select_attn_kernel<true>, grid, dim3(kSelWaves * 64), lds, stream, q, k_cmp, k, v,
                       blk_idx, blk_score, out, lse, part, s);
  else
    hipLaunchKernelGGL(decode_select_attn_kernel<false>, grid, dim3(kSelWaves * 64), lds, stream, q, k_cmp, k, v,
                       blk_idx, blk_score, out, lse, part, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || s.nsplit == 1) return err;
  return launch_combine_splits(part, out, lse, s, stream);
}

template <int R>
static hipError_t launch_select_r(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx, float* blk_score,
                                  const AttnShape& s, hipStream_t stream) {
  auto grid = [&](int tok) { return dim3((s.S_q + tok - 1) / tok, s.B * s.H_kv); };
  if (select_lds<64, kSelWideWaves>(s.NB) <= kSelLdsMax / 2) {
    // up to 512 blocks: 8-token workgroups, two per CU (32k: 0.329 -> 0.287 ms)
    hipLaunchKernelGGL((select_blocks_kernel<64, R, kSelWideWaves, 2>), grid(kSelWideWaves),
                       dim3(64 * kSelWideWaves), (select_lds<64, kSelWideWaves>(s.NB)), stream, q, k_cmp, blk_idx,
                       blk_score, s);
  } else if (select_lds<64, kSelWideWaves, 2>(s.NB) <= kSelLdsMax / 2) {
    // up to 1536 blocks: the same with one 64-block chunk at a time, so that
    // two workgroups' score rows fit (64k: 1.00 -> 0.94 ms against 16-token
    // workgroups of chunk pairs)
    hipLaunchKernelGGL((select_blocks_kernel<64, R, kSelWideWaves, 2, 2>), grid(kSelWideWaves),
                       dim3(64 * kSelWideWaves), (select_lds<64, kSelWideWaves, 2>(s.NB)), stream, q, k_cmp, blk_idx,
                       blk_score, s);
  } else if (select_lds<32, kSelWideWaves, 2>(s.NB) <= kSelLdsMax / 2) {
    // up to 2048 blocks: 8-token workgroups, two per CU, one 32-block chunk at
    // a time (128k: 3.68 -> 3.44 ms against 16-token workgroups of chunk pairs)
    hipLaunchKernelGGL((select_blocks_kernel<32, R, kSelWideWaves, 2, 2>), grid(kSelWideWaves),
                       dim3(64 * kSelWideWaves), (select_lds<32, kSelWideWaves, 2>(s.NB)), stream, q, k_cmp, blk_idx,
                       blk_score, s);
  } else {  // 2049 .. 4064 blocks: 8-token workgroups, one per CU
    hipLaunchKernelGGL((select_blocks_kernel<32, R, kSelWideWaves>), grid(kSelWideWaves), dim3(64 * kSelWideWaves),
                       (select_lds<32, kSelWideWaves>(s.NB)), stream, q, k_cmp, blk_idx, blk_score, s);
  }
  return hipGetLastError();
}

hipError_t launch_select_blocks(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx,
                                float* blk_score, const AttnShape& s, hipStream_t stream, int lse_stride) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  if (s.S_q == 1 && lse_stride == 1 && s.NB <= kSelWaves * kDecTiles * 16) {
    // one query per sequence: the workgroup splits its blocks
    const size_t lds = decode_select_lds(s.NB);
    hipLaunchKernelGGL(select_decode_kernel, dim3(s.B * s.H_kv), dim3(64 * kSelWaves), lds, stream, q, k_cmp,
                       blk_idx, blk_score, s);
    return hipGetLastError();
  }
  switch (lse_stride) {
    case 2: return launch_select_r<2>(q, k_cmp, blk_idx, blk_score, s, stream);
    case 4: return launch_select_r<4>(q, k_cmp, blk_idx, blk_score, s, stream);
    case 8: return launch_select_r<8>(q, k_cmp, blk_idx, blk_score, s, stream);
    default: return launch_select_r<1>(q, k_cmp, blk_idx, blk_score, s, stream);
  }
}

}  // namespace infv2
