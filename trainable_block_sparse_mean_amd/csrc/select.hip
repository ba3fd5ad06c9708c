// Block selection: group-summed block scores + top-k.
//
// Scores: skill page "Infllm V2 Dense Sparse Switchable Attention",
// Architecture Overview (Hardware Kernel: log-sum-exp-normalised scores
// summed over the heads of a group) and Step 2 (compressed_attention: softmax
// of the scaled query / compressed-key products).  Selection: Step 2,
// selected_attention (top-k per query position) at block granularity (news
// summary, Technical Mechanism).
//
// One workgroup = 16 consecutive query tokens of one KV head, one token per
// wave.  The compressed keys stream through a 3-slot LDS ring of CH-block
// chunks (direct-to-LDS loads, two chunks in flight, one barrier per chunk)
// that all 16 waves read, so each chunk comes from L2 once per workgroup and
// pass.  For a token, S = Q k_cmp^T on 16x16x32 bf16 MFMAs puts the 16 heads
// of the group in the rows and 16 compressed blocks in the columns: lane
// (column hl, row quad gq) holds heads 4*gq .. 4*gq+3 of block 16*tile + hl.
//   pass 1: each lane keeps, per head, a running max (moved only when a
//           score exceeds it by 2^8) and a sum of exp2 over its blocks; the 16
//           lanes of a row are merged at the end -> per-head log-sum-exp
//           (log2 units).
//   pass 2: p = exp2(z - lse) per head, the group score of a block is the sum
//           over the lane's 4 heads and the 4 row quads (two permlane swaps);
//           it goes to LDS only, never to HBM.
// Heads beyond G (G < 16) have zero queries and an infinite log-sum-exp, so
// they add exactly 0.  The top-k is an exact radix select on the fp32 bit
// patterns (non-negative floats order like their bits); ties are then taken
// lowest index first and the kept indices compacted in ascending order by
// ballot.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kSelWaves = 16;           // = tokens per workgroup
constexpr int kSelSlots = 3;            // LDS ring: the chunk being read + 2 in flight
constexpr int kSelRowBytes = kD * 2;    // one compressed block
constexpr size_t kSelLdsMax = 160 * 1024;
constexpr float kSelSlack = 8.f;         // log2 units a running max may lag

// floats per token row of block scores in LDS
__host__ __device__ constexpr int sel_stride(int NB) { return (NB + 3) & ~3; }

template <int CH>
constexpr size_t select_lds(int NB) {
  return static_cast<size_t>(kSelSlots) * CH * kSelRowBytes + static_cast<size_t>(kSelWaves) * sel_stride(NB) * 4;
}

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

// Exact top-kk (kk = topk < nC) of the nC scores cand[0 .. nC), candidate c
// in slot c / 64 of lane c % 64 (NS >= ceil(nC / 64) slots per lane).  Keys
// are the fp32 bit patterns with the sign cleared: every key is below 2^31,
// also for NaN scores (which order above +inf), and non-negative floats order
// like their keys.  A bitwise radix search finds a threshold tt: the kk-th
// largest key, or any prefix of it at or below which exactly kk keys lie.
// The keys above tt and the first (lowest-index) ties at tt are kept, written
// to out[0 .. kk) in ascending index order (index = first + c).
template <int NS>
__device__ __forceinline__ void topk_row(const float* cand, int nC, int topk, int first, int32_t* out,
                                         float* out_s, int lane) {
  const int kk = topk;
  uint32_t x[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int c = t * 64 + lane;
    x[t] = c < nC ? __float_as_uint(cand[c]) & 0x7fffffffu : 0u;
  }
  // largest tt with #{x >= tt} >= kk (padding keys are 0 and never reach a
  // candidate value, which has a bit set).  The search may stop as soon as
  // exactly kk keys are >= the prefix found so far: those kk keys are then
  // the selection, and the pass below keeps exactly them.
  uint32_t tt = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cv = tt | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int t = 0; t < NS; ++t) cnt += __popcll(__ballot(x[t] >= cv));
    if (cnt >= kk) {
      tt = cv;
      if (cnt == kk) break;
    }
  }
  int n_gt = 0;
#pragma unroll
  for (int t = 0; t < NS; ++t) n_gt += __popcll(__ballot(x[t] > tt));
  const int need_eq = kk - n_gt;  // ties at tt, lowest indices first

  int eq_before = 0, n_out = 0;
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const bool valid = t * 64 + lane < nC;
    const bool gt = x[t] > tt;
    const bool eq = valid && x[t] == tt;
    const uint64_t eqm = __ballot(eq);
    const bool sel = gt || (eq && eq_before + mask_rank(eqm) < need_eq);
    eq_before += __popcll(eqm);
    const uint64_t selm = __ballot(sel);
    const int pos = n_out + mask_rank(selm);
    if (sel && pos < kk) {
      out[pos] = first + t * 64 + lane;
      if (out_s) out_s[pos] = __uint_as_float(x[t]);
    }
    n_out += __popcll(selm);
  }
}

// R = 1: exact log-sum-exp in pass 1.  R > 1: the approximate one of
// infv2_select_blocks_strided_lse - pass 1 scores only every R-th visible
// compressed block, each standing for the R blocks of its group (the last
// group for its visible count), so it streams 1/R of the compressed keys.
template <int CH, int R>
__global__ __launch_bounds__(kSelWaves * 64) void select_blocks_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ kc,
                                                                       int32_t* __restrict__ blk_idx,
                                                                       float* __restrict__ blk_score,
                                                                       AttnShape s) {
  constexpr int kTiles = CH / 16;               // 16-block MFMA tiles per chunk
  constexpr int kSlotBytes = CH * kSelRowBytes;
  constexpr int kDmaWaves = CH / 4;             // each moves 4 rows (1 KB) of a chunk
  extern __shared__ __align__(16) unsigned char sel_smem[];
  const uint32_t ring = lds_addr(sel_smem);
  float* sig_all = reinterpret_cast<float*>(sel_smem + kSelSlots * kSlotBytes);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar) from here on
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15;   // MFMA column: block within the tile
  const int gq = lane >> 4;   // row quad: heads 4*gq .. 4*gq+3
  const int g = blockIdx.y % s.H_kv;
  const int b = blockIdx.y / s.H_kv;
  const int r0 = (gridDim.x - 1 - blockIdx.x) * kSelWaves;  // latest (heaviest) tokens first
  const int r = r0 + wave;    // this wave's token
  const int off = seq_keys(s, b) - s.S_q;  // query row r sits at key position off + r
  const bool active = r < s.S_q;
  const int nv = active ? (off + r + 1) / kBS : 0;  // fully visible blocks
  const int r_last = min(r0 + kSelWaves, s.S_q) - 1;
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

  // chunk loads: wave w < kDmaWaves moves rows 4w .. 4w+3 of a chunk; lane
  // (sub, slot) fetches 16-byte column slot ^ swz(row) of row 4w + sub into
  // that row's slot (rows past NB - 1 re-read row NB - 1; never used)
  const int drow = 4 * wave + (lane >> 4);
  const uint32_t dcol = static_cast<uint32_t>(((lane & 15) ^ swz(drow)) << 4);
  const int nit = nch1 + nch;  // pass 1 chunks, then pass 2 chunks
  auto stage = [&](int it) {
    if (wave < kDmaWaves && it < nit) {
      const int j = min(it < nch1 ? R * (it * CH + drow) : (it - nch1) * CH + drow, s.NB - 1);
      dma16(kg, static_cast<uint32_t>(j) * kSelRowBytes + dcol,
            ring + (it % kSelSlots) * kSlotBytes + wave * 1024);
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
  // than kSelSlack (decided per wave), so most chunks need no rescaling; the
  // sum stays below 2^8 per term.
  auto lse_update = [&](const floatx4* acc, auto nt_c) {
    constexpr int NT = decltype(nt_c)::value;
    float mx[4];
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx[i] = acc[0][i];
#pragma unroll
      for (int t = 1; t < NT; ++t) mx[i] = fmaxf(mx[i], acc[t][i]);
      mx[i] *= sl2;
      need |= mx[i] > m[i] + kSelSlack;
    }
    if (__ballot(need) != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mn = fmaxf(m[i], mx[i]);
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
  auto group_score = [&](const floatx4& acc) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) p += __builtin_amdgcn_exp2f(fmaf(acc[i], sl2, -lse2[i]));
    return sum_xor32(sum_xor16(p));
  };
  using AllTiles = std::integral_constant<int, kTiles>;
  using OneTile = std::integral_constant<int, 1>;

  stage(0);
  stage(1);
  for (int it = 0; it < nit; ++it) {  // pass 1 chunks, then pass 2 chunks
    if (it + 1 < nit) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // chunk `it` is in LDS; every wave is done with chunk it - 1
    stage(it + 2);    // into the slot chunk it - 1 used
    if (it == nch1) {
      // end of pass 1: merge the 16 lanes of each row (one head per register i)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lse_merge_row<0x128>(m[i], l[i]);
        lse_merge_row<0x124>(m[i], l[i]);
        lse_merge_row<0x122>(m[i], l[i]);
        lse_merge_row<0x121>(m[i], l[i]);
        lse2[i] = 4 * gq + i < s.G ? m[i] + log2f(l[i]) : INFINITY;
      }
    }
    const unsigned char* buf = sel_smem + (it % kSelSlots) * kSlotBytes;
    if (it < nch1) {
      // pass 1 over rows jc .. jc + CH - 1 of the sampled sequence: sampled
      // row x is block R * x, standing for blocks R*x .. R*x + R-1 that are
      // visible (weight w: log2(w) / sl2 added to its scores)
      const int jc = it * CH;
      if (!active || R * jc >= nv) continue;
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
      continue;
    }
    const int jc = (it - nch1) * CH;  // first block of the pass 2 chunk
    if (!active || jc >= nv) continue;
    const bool full = jc + CH <= nv;
    {
      if (full) {
        floatx4 acc[kTiles];
        scores(buf, 0, AllTiles{}, acc);
        // row quad gq stores tile gq % kTiles (quads with the same tile store
        // the same value to the same address)
        float mine = 0.f;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const float p = group_score(acc[t]);
          mine = (gq % kTiles) == t ? p : mine;
        }
        sig[jc + 16 * (gq % kTiles) + hl] = mine;
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
  const int nIt = (nC + 63) / 64;  // candidate slots per lane (<= 32)
  if (nIt <= 1) topk_row<1>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 2) topk_row<2>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 4) topk_row<4>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 8) topk_row<8>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 16) topk_row<16>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else topk_row<32>(sig + lo, nC, s.topk, lo, out, out_s, lane);
}

// One query per sequence (decode): the 16 waves of a workgroup share the
// token and split its visible compressed blocks, so the whole workgroup works
// on one selection.  Wave w scores the 16-block tiles [w*tpw, (w+1)*tpw), its
// compressed keys loaded straight into the B operands (each block is read by
// one wave only, so nothing is staged in LDS), and keeps the scores in
// registers: the two passes become one pass over the keys.  The waves' (max,
// sum) per head are merged in LDS into the exact log-sum-exp, each wave turns
// its own scores into group scores in LDS, and wave 0 takes the top-k as the
// token-per-wave kernel does.  Same lane layout as that kernel.
constexpr int kDecTiles = 8;  // tiles per wave: 16 waves x 8 x 16 blocks covers 2048 blocks
__global__ __launch_bounds__(kSelWaves * 64) void select_decode_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ kc,
                                                                       int32_t* __restrict__ blk_idx,
                                                                       float* __restrict__ blk_score, AttnShape s) {
  extern __shared__ __align__(16) unsigned char dec_smem[];
  float* part = reinterpret_cast<float*>(dec_smem);              // [16 waves][16 heads][2]
  float* sig = part + kSelWaves * kMaxG * 2;                        // [NB]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15, gq = lane >> 4;
  const int g = blockIdx.x % s.H_kv;
  const int b = blockIdx.x / s.H_kv;
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
  // the query and the first two tiles' keys are loaded together
  u32x4 kra[4], krb[4];
  if (tw0 < tend) kload(0, kra);
  if (tw0 + 1 < tend) kload(1, krb);
  bf16x8 qa[4];
  {
    const bool ok = hl < s.G;
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q) * kD + gq * 8;
    u32x4 raw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) raw[ks] = ok ? load16(qrow + ks * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = settle(as_bf16x8(raw[ks]));
  }

  // scores of this wave's tiles (log2 units); blocks >= nv are -inf.  Tiles go
  // in pairs, the next pair's keys loaded under the current pair's products.
  floatx4 z[kDecTiles];
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int t = 0; t < kDecTiles; ++t) m[i] = fmaxf(m[i], z[t][i]);
    if (m[i] != -INFINITY) {
#pragma unroll
      for (int t = 0; t < kDecTiles; ++t) l[i] += __builtin_amdgcn_exp2f(z[t][i] - m[i]);
    }
    // the 16 lanes of the row hold the same head's other blocks
    lse_merge_row<0x128>(m[i], l[i]);
    lse_merge_row<0x124>(m[i], l[i]);
    lse_merge_row<0x122>(m[i], l[i]);
    lse_merge_row<0x121>(m[i], l[i]);
    if (hl == 0) {
      part[(wave * kMaxG + 4 * gq + i) * 2] = m[i];
      part[(wave * kMaxG + 4 * gq + i) * 2 + 1] = l[i];
    }
  }
  __syncthreads();
  float lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * gq + i;
    float mm = -INFINITY;
    for (int w = 0; w < kSelWaves; ++w) mm = fmaxf(mm, part[(w * kMaxG + h) * 2]);
    float ll = 0.f;
    for (int w = 0; w < kSelWaves; ++w) {
      const float mw = part[(w * kMaxG + h) * 2];
      if (mw != -INFINITY) ll += part[(w * kMaxG + h) * 2 + 1] * exp2f(mw - mm);
    }
    lse2[i] = h < s.G && mm != -INFINITY ? mm + log2f(ll) : INFINITY;  // heads >= G add nothing
  }
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
  if (wave != 0 || s.topk == 0) return;

  const int qb = pos / kBS;
  const int lo = s.n_init;
  const int hi = qb - s.n_local;
  const int nC = hi >= lo ? hi - lo + 1 : 0;
  int32_t* out = blk_idx + static_cast<size_t>(b * s.H_kv + g) * s.S_q * s.topk;
  float* out_s = blk_score ? blk_score + static_cast<size_t>(b * s.H_kv + g) * s.S_q * s.topk : nullptr;
  if (nC <= s.topk) {
    for (int e = lane; e < s.topk; e += 64) {
      out[e] = e < nC ? lo + e : -1;
      if (out_s) out_s[e] = e < nC ? sig[lo + e] : 0.f;
    }
    return;
  }
  const int nIt = (nC + 63) / 64;
  if (nIt <= 1) topk_row<1>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 2) topk_row<2>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 4) topk_row<4>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 8) topk_row<8>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else if (nIt <= 16) topk_row<16>(sig + lo, nC, s.topk, lo, out, out_s, lane);
  else topk_row<32>(sig + lo, nC, s.topk, lo, out, out_s, lane);
}

template <int R>
static hipError_t launch_select_r(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx, float* blk_score,
                                  const AttnShape& s, hipStream_t stream) {
  dim3 grid((s.S_q + kSelWaves - 1) / kSelWaves, s.B * s.H_kv);
  // 64-block chunks where the LDS holds them, else 32 (NB <= 2048 fits)
  if (select_lds<64>(s.NB) <= kSelLdsMax)
    hipLaunchKernelGGL((select_blocks_kernel<64, R>), grid, dim3(64 * kSelWaves), select_lds<64>(s.NB), stream, q,
                       k_cmp, blk_idx, blk_score, s);
  else
    hipLaunchKernelGGL((select_blocks_kernel<32, R>), grid, dim3(64 * kSelWaves), select_lds<32>(s.NB), stream, q,
                       k_cmp, blk_idx, blk_score, s);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx,
                                float* blk_score, const AttnShape& s, hipStream_t stream, int lse_stride) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  if (s.S_q == 1 && lse_stride == 1) {  // one query per sequence: the workgroup splits its blocks
    const size_t lds = (static_cast<size_t>(kSelWaves) * kMaxG * 2 + sel_stride(s.NB)) * sizeof(float);
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
