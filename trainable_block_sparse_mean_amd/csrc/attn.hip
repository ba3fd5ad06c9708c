// Block-sparse and dense attention forward for gfx950.
//
// Sparse: news summary "Technical Mechanism" (attention only on the selected
// key-value blocks) plus the initial blocks and a causal block-granular
// sliding window (skill page "Infllm V2 Dense Sparse Switchable Attention",
// Step 2 sliding_attention, made causal per Practical Guidance, When NOT to
// Use).  Dense: skill page, Step 1 (softmax of scaled products, weighted sum
// of values).
//
// Work unit: one workgroup = one KV head of one batch entry x a window of
// W = 16 consecutive query tokens.  Sparse: 16 waves of one token each (four
// per SIMD, every member token an independent instruction stream).  Dense:
// 8 waves of two tokens each.  The G <= 16 query heads of the KV head share
// every K/V byte.
//   * The sparse workgroup builds the union of the blocks its tokens attend
//     (a per-block bitmask of member tokens in LDS, compacted to an ascending
//     list) and streams each block of the union once through LDS, two blocks
//     per barrier; few query windows (decode) split the list over several
//     workgroups whose partial results a second kernel merges.
//   * K and V blocks go global -> LDS with asynchronous direct-to-LDS loads
//     (global_load_lds_dwordx4) into a 4-stage ring.  LDS rows are 256 bytes
//     whose 16-byte chunks are permuted by a linear swizzle of the row, which
//     keeps every fragment read pattern below free of bank conflicts.
//   * Scores are computed transposed, S^T = K Q^T (keys x heads): each lane
//     then owns one head and a few keys, the row max needs only cross-lane
//     swaps (v_permlane{16,32}_swap), and the softmax output is already the
//     B operand of O^T += V^T P^T once the keys of a k-step are taken in the
//     order the lanes hold them.  The matching V^T operand comes straight
//     from V's natural [key][dim] rows through the transposing LDS read
//     ds_read_b64_tr_b16 (each 16-lane group turns a 4-key x 16-dim tile into
//     one 4-key column per lane).
//   * Sparse: one token per MFMA column block (16x16x32 bf16, N = 16 heads),
//     so a token that does not attend a block costs nothing.  Dense: every
//     token attends every earlier block, so the two tokens of a wave share a
//     32x32x16 bf16 MFMA (N = 2 tokens x 16 heads) and every K/V fragment
//     read from LDS serves both.
//   * Online softmax in log2 units; the running max only moves when a block
//     max exceeds it by more than 2^8, so the O rescale is rare.
#include "attn_common.hpp"

namespace infv2 {

// Sparse: 16 waves x 1 token (4 waves per SIMD: every member token is an
// independent instruction stream).  Dense: 8 waves x 2 tokens (the 32 MFMA
// columns).  Both cover a window of kWin = 16 tokens.
template <bool DENSE> struct Cfg;
template <> struct Cfg<false> { static constexpr int kTok = 1, kWaves = 16; };
template <> struct Cfg<true> { static constexpr int kWaves = 8, kTok = 2; };
// ---------------------------------------------------------------------------
// Dense: 32x32x16 MFMAs, the wave's two tokens side by side in the 32
// columns (lane column c32 = 16 * token + head, key/dim half h2).
// ---------------------------------------------------------------------------
struct DenseState {
  bf16x8 qf[8];        // Q^T B operands, k-steps of 16 dims
  floatx16 o[4];       // O^T accumulators, 4 tiles of 32 dims
  float m, l;
  int lim;             // last visible key position of this lane's token
};

// Per-lane LDS byte offsets of the dense fragment reads within a stage: K
// for k-step ks at row c32 (+32 rows per key tile); V (transposing reads)
// for dim tile dt and half hh at row 8*hh + 4*h2 + li/4 (+16 rows per k-step).
struct DenseLane {
  uint32_t k[8], v[4][2];
};
__device__ __forceinline__ DenseLane dense_lane(int lane) {
  DenseLane o;
  const int c32 = lane & 31, h2 = lane >> 5, grp = lane >> 4, li = lane & 15;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) o.k[ks] = c32 * kRowBytes + (((2 * ks + h2) ^ swz(c32)) << 4);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int vr = 8 * hh + 4 * h2 + (li >> 2);
      const int chunk = 4 * dt + 2 * (grp & 1) + ((li & 3) >> 1);
      o.v[dt][hh] = vr * kRowBytes + ((chunk ^ swz(vr)) << 4) + ((li & 1) << 3);
    }
  return o;
}

__device__ __forceinline__ void dense_block(DenseState& st, const DenseLane& ln, const unsigned char* kbuf,
                                            const unsigned char* vbuf, int j, float sl2, bool need_mask, int h2) {
  // S^T tile kt: rows = keys 32*kt + 8*(i/4) + 4*h2 + i%4 of accumulator value i
  floatx16 sacc[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    floatx16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = mfma_32x32x16(as_bf16x8(load16(kbuf + ln.k[ks] + kt * 32 * kRowBytes)), st.qf[ks], acc);
    sacc[kt] = acc;
  }
  if (need_mask) {  // wave-uniform: the block reaches past one of the tokens
    const int first = st.lim - j * kBS - 4 * h2;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kt + 8 * (i >> 2) + (i & 3) > first) sacc[kt][i] = -INFINITY;
  }
  float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mx0 = fmaxf(mx0, sacc[0][i]);
    mx1 = fmaxf(mx1, sacc[1][i]);
  }
  const float mx = max_xor32(fmaxf(mx0, mx1)) * sl2;
  const bool grow = mx > st.m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mn = grow ? mx : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] *= alpha;
    st.m = mn;
  }
  const float nm = -st.m;
  // P^T k-step s (keys 16*s .. 16*s+15): values 8*(s%2) .. 8*(s%2)+7 of tile s/2
  bf16x8 pf[4];
  float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][8 * (s & 1) + 2 * e], sl2, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][8 * (s & 1) + 2 * e + 1], sl2, nm));
      pw[e] = pack_bf16x2(p0, p1);
      rs0 += p0;
      rs1 += p1;
    }
    pf[s] = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
  }
  st.l += rs0 + rs1;
  // O^T += V^T P^T; k-step s, slot e of half h2 is key 16*s + 8*(e/4) + 4*h2 + e%4,
  // dim 32*dt + c32: two transposing reads of 4-key x 16-dim tiles
  // k-step outer, dim tile inner: 4 independent MFMAs per step
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 vf[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      vf[dt] = __builtin_shufflevector(lds_read_tr(vbuf + ln.v[dt][0] + s * 16 * kRowBytes),
                                       lds_read_tr(vbuf + ln.v[dt][1] + s * 16 * kRowBytes), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] = mfma_32x32x16(vf[dt], pf[s], st.o[dt]);
  }
}

// The compressed-attention branch of the mixed launch (see launch_mixed_attn)
struct MixArgs {
  const uint16_t* kc;  // compressed keys / values [B][H_kv][NB][D]
  const uint16_t* vc;
  float w_sparse, w_cmp;
};

// List entry e of the compressed branch: group e (compressed rows 64e ..
// 64e+63) | the window's tokens that see its first row (token t of a window
// of nq tokens from query row r0, key position off + r0 + t, sees row 64e iff
// off + r0 + t + 1 >= 64 (64e + 1)).
__device__ __forceinline__ uint32_t cmp_entry(int e, int off, int r0, int nq) {
  const int t_min = max(0, kBS * (kBS * e + 1) - 1 - off - r0);
  const uint32_t mask = t_min >= nq ? 0u : ((1u << nq) - 1u) & ~((1u << t_min) - 1u);
  return static_cast<uint32_t>(e) | (mask << 16);
}

// PAGED: K/V in the pages of a paged cache, per-sequence lengths (decode);
// otherwise contiguous K/V of one key length.  MIX: the compressed branch runs
// first on the same pipeline and the epilogue mixes it into the output.
template <bool DENSE, bool PAGED, bool MIX>
__global__ __launch_bounds__(Cfg<DENSE>::kWaves * 64, 1) void attn_window_kernel(const uint16_t* __restrict__ q,
                                                                     const uint16_t* __restrict__ k,
                                                                     const uint16_t* __restrict__ v,
                                                                     const int32_t* __restrict__ blk_idx,
                                                                     uint16_t* __restrict__ out,
                                                                     float* __restrict__ lse,
                                                                     float* __restrict__ part, AttnShape s,
                                                                     MixArgs mx) {
  static_assert(!MIX || (!DENSE && !PAGED), "the mix runs on the contiguous sparse path");
  constexpr int kWaves = Cfg<DENSE>::kWaves;
  constexpr int T = Cfg<DENSE>::kTok;
  constexpr int NT = kWaves * 64;
  extern __shared__ __align__(1024) unsigned char smem[];
  uint32_t* bmask = reinterpret_cast<uint32_t*>(smem + kStages * kStageBytes);  // [NB], sparse only
  int* blist = reinterpret_cast<int*>(bmask + s.NB);                           // [NB], sparse only
  int* n_list = blist + s.NB;                                                  // list length, sparse only

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nwin = (s.S_q + kWin - 1) / kWin;
  int bg_i, win;
  if (!map_window(blockIdx.x, nwin, s.B * s.H_kv, bg_i, win)) return;
  const int g = bg_i % s.H_kv;
  const int b = bg_i / s.H_kv;
  const size_t bg = static_cast<size_t>(bg_i);
  const int r0 = win * kWin;
  const int rw = r0 + wave * T;              // first token of this wave
  const int S_k = PAGED ? seq_keys(s, b) : s.S_k;  // keys of this sequence
  const int off = S_k - s.S_q;
  const int i_last = off + min(r0 + kWin, s.S_q) - 1;
  const int qb_last = i_last / kBS;
  const uint16_t* kg = PAGED ? k : k + bg * s.S_k * kD;  // pages, or this KV head's contiguous rows
  const uint16_t* vg = PAGED ? v : v + bg * s.S_k * kD;
  const BlockSrc<PAGED> src{kg, vg, s.block_table, s.NB, s.num_pages, s.H_kv, b, g, S_k};
  const uint32_t ring = lds_addr(smem);
  const float sl2 = s.scale_log2;

  // ---- per-token queries (the compiler waits for them once, in settle) -----
  SparseState sp[T];  // sparse: one state per token of the wave
  DenseState dn;
  if constexpr (DENSE) {
    const int c32 = lane & 31, h2 = lane >> 5;
    const int tok = c32 >> 4, hd = c32 & 15;
    const int r = rw + tok;
    const bool valid = r < s.S_q && hd < s.G;
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + g * s.G + hd) * s.S_q + r) * kD + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) dn.qf[ks] = valid ? as_bf16x8(load16(qrow + 16 * ks)) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) dn.qf[ks] = settle(dn.qf[ks]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dn.o[dt] = floatx16{};
    dn.m = -INFINITY;
    dn.l = 0.f;
    dn.lim = s.causal ? min(off + r, S_k - 1) : S_k - 1;
  } else {
    const int hl = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int r = rw + t;
      const bool valid = r < s.S_q && hl < s.G;
      const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q + r) * kD + gq * 8;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sp[t].qf[ks] = valid ? as_bf16x8(load16(qrow + ks * 32)) : bf16x8{};
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sp[t].qf[ks] = settle(sp[t].qf[ks]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) sp[t].o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      sp[t].m = -INFINITY;
      sp[t].l = 0.f;
      sp[t].lim = min(off + rw + t, S_k - 1);
    }
  }

  // ---- the union of attended blocks ---------------------------------------
  // Sparse: list entry = block index | (16-bit member mask of the window's
  // tokens) << 16, ascending by block.
  int nblk;
  if constexpr (DENSE) {
    nblk = s.causal ? qb_last + 1 : s.NB;
  } else {
    nblk = build_union_list<NT>(bmask, blist, n_list, blk_idx, bg, r0, off, qb_last, s, wave, lane);
    if constexpr (MIX) {
      // The compressed branch first, streamed like a block list (64
      // compressed rows side by side have a key block's layout; the token
      // sees rows 0 .. nv-1): its output times w_cmp goes to out, which the
      // epilogue reads back.  Then the state restarts for the sparse part.
      static_assert(T == 1, "one token per wave");
      const int hl = lane & 15, gq = lane >> 4;
      const int nq = min(kWin, s.S_q - r0);
      const int ngrp = ((off + r0 + nq) / kBS + kBS - 1) / kBS;
      const BlockSrc<false> csrc{mx.kc + bg * s.NB * kD, mx.vc + bg * s.NB * kD, nullptr, s.NB, 0, s.H_kv, b, g,
                                 s.NB};
      sp[0].lim = (off + rw + 1) / kBS - 1;  // last visible compressed row (-1: none)
      const SparseLane cspl = sparse_lane(hl, gq);
      stream_pairs<kWaves>(smem, csrc, 0, ngrp, [&](int e) { return cmp_entry(e, off, r0, nq); }, wave, lane,
                           [&](const unsigned char* const* stg, const int* js, uint32_t cur0, uint32_t cur1) {
        const uint32_t bit = 1u << (16 + wave);
        attend_pair(sp[0], cspl, stg, js, (cur0 & bit) != 0u, (cur1 & bit) != 0u, lane, sl2);
      });
      const float l = sum_xor32(sum_xor16(sp[0].l));
      if (rw < s.S_q && hl < s.G) {
        const float scl = l > 0.f ? mx.w_cmp / l : 0.f;  // no visible block: the branch is zero
        uint16_t* orow = out + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q + rw) * kD + 4 * gq;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<u32x2*>(orow + 16 * dt) = u32x2{pack_bf16x2(sp[0].o[dt][0] * scl, sp[0].o[dt][1] * scl),
                                                           pack_bf16x2(sp[0].o[dt][2] * scl, sp[0].o[dt][3] * scl)};
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) sp[0].o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      sp[0].m = -INFINITY;
      sp[0].l = 0.f;
      sp[0].lim = min(off + rw, S_k - 1);
      __syncthreads();  // every wave is done with the ring
    }
  }
  // entry e of the list (dense: every block in order)
  auto entry_at = [&](int e) -> uint32_t {
    if constexpr (DENSE) return static_cast<uint32_t>(e);
    else return e < nblk ? static_cast<uint32_t>(blist[e]) : 0u;
  };

  const DmaLane<kWaves> dl = dma_lane<kWaves>(wave, lane);
  constexpr int kDma = 2 * DmaLane<kWaves>::kChunks;  // loads per wave per block

  if constexpr (DENSE) {
    // prologue: the first kStages - 1 blocks in flight
#pragma unroll
    for (int e = 0; e < kStages - 1; ++e)
      if (e < nblk) stage_src(ring + e * kStageBytes, src, e, dl, wave, lane);
    // this wave's two tokens' visibility limits (a token past the end of the
    // queries takes its partner's)
    const int lim0 = s.causal ? min(off + rw, S_k - 1) : S_k - 1;
    const int lim1 = rw + 1 < s.S_q ? (s.causal ? min(off + rw + 1, S_k - 1) : S_k - 1) : lim0;
    const DenseLane dnl = dense_lane(lane);
    for (int j = 0; j < nblk; ++j) {
      wait_dma<kDma>(min(kStages - 2, nblk - 1 - j));
      __syncthreads();  // block j is in LDS; every wave is done with block j - 1
      if (j + kStages - 1 < nblk)
        stage_src(ring + ((j + kStages - 1) % kStages) * kStageBytes, src, j + kStages - 1, dl, wave, lane);
      if (rw >= s.S_q || j * kBS > lim1) continue;   // neither token sees block j
      const unsigned char* kbuf = smem + (j % kStages) * kStageBytes;
      dense_block(dn, dnl, kbuf, kbuf + kTileBytes, j, sl2, j * kBS + kBS - 1 > lim0, lane >> 5);
    }
  } else {
    // Pairs of list entries, one barrier per pair (stream_pairs).
    const SparseLane spl = sparse_lane(lane & 15, lane >> 4);
    // split-KV: this workgroup takes entries [e_lo, e_hi) of the list
    const int split = blockIdx.y;
    const int e_lo = static_cast<int>(static_cast<long long>(split) * nblk / s.nsplit);
    const int e_hi = static_cast<int>(static_cast<long long>(split + 1) * nblk / s.nsplit);
    stream_pairs<kWaves, false, 8>(smem, src, e_lo, e_hi, entry_at, wave, lane,
                         [&](const unsigned char* const* stg, const int* js, uint32_t cur0, uint32_t cur1) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t bit = 1u << (16 + wave * T + t);   // cur1 = 0 past the list
        attend_pair(sp[t], spl, stg, js, (cur0 & bit) != 0u, (cur1 & bit) != 0u, lane, sl2);
      }
    });
  }

  // ---- epilogue ---------------------------------------------------------------
  if constexpr (DENSE) {
    const int c32 = lane & 31, h2 = lane >> 5;
    const int tok = c32 >> 4, hd = c32 & 15;
    const int r = rw + tok;
    const float l = sum_xor32(dn.l);
    if (r < s.S_q && hd < s.G) {
      const int h = g * s.G + hd;
      const float inv = 1.f / l;
      uint16_t* orow = out + (static_cast<size_t>(b * s.H_q + h) * s.S_q + r) * kD + 4 * h2;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x2 w = {pack_bf16x2(dn.o[dt][4 * a] * inv, dn.o[dt][4 * a + 1] * inv),
                           pack_bf16x2(dn.o[dt][4 * a + 2] * inv, dn.o[dt][4 * a + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a) = w;
        }
      if (lse && h2 == 0) lse[static_cast<size_t>(b * s.H_q + h) * s.S_q + r] = (dn.m + log2f(l)) * kLn2;
    }
  } else {
    const int hl = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int r = rw + t;
      const float l = sum_xor32(sum_xor16(sp[t].l));
      if (r >= s.S_q || hl >= s.G) continue;
      const int h = g * s.G + hl;
      if (s.nsplit > 1) {
        // unnormalised partial state of this split, merged by combine_splits_kernel
        float* pr = part + ((static_cast<size_t>(blockIdx.y) * s.B * s.H_q + b * s.H_q + h) * s.S_q + r) * kPartFloats;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<floatx4*>(pr + 16 * dt + 4 * gq) = sp[t].o[dt];
        if (gq == 0) {
          pr[128] = sp[t].m;
          pr[129] = l;
        }
        continue;
      }
      const float inv = MIX ? mx.w_sparse / l : 1.f / l;
      uint16_t* orow = out + (static_cast<size_t>(b * s.H_q + h) * s.S_q + r) * kD + 4 * gq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = sp[t].o[dt][e] * inv;
        if constexpr (MIX) {  // this lane wrote these four values in the branch phase
          const u32x2 c = *reinterpret_cast<const u32x2*>(orow + 16 * dt);
          y[0] += bf16_lo(c[0]);
          y[1] += bf16_hi(c[0]);
          y[2] += bf16_lo(c[1]);
          y[3] += bf16_hi(c[1]);
        }
        const u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2*>(orow + 16 * dt) = w;
      }
      if (lse && gq == 0) lse[static_cast<size_t>(b * s.H_q + h) * s.S_q + r] = (sp[t].m + log2f(l)) * kLn2;
    }
  }
}

// Merge the split partials of each query row: m = max_s m_s,
// l = sum_s l_s 2^(m_s - m), O = sum_s o_s 2^(m_s - m) / l.  One workgroup of
// 128 threads (one per dim) per row.  Every split's values are loaded up front
// (unrolled to the largest split count), so the row waits on one round of
// loads rather than on one per split.
constexpr int kMaxSplits = 16;  // sparse_splits never returns more
__global__ __launch_bounds__(128) void combine_splits_kernel(const float* __restrict__ part,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse,
                                                             int nsplit, size_t rows) {
  const size_t row = blockIdx.x;
  const int d = threadIdx.x;
  const size_t stride = rows * kPartFloats;
  const float* pr = part + row * kPartFloats;
  float ms[kMaxSplits], ls[kMaxSplits], os[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    const bool ok = sp < nsplit;
    ms[sp] = ok ? pr[sp * stride + 128] : -INFINITY;
    ls[sp] = ok ? pr[sp * stride + 129] : 0.f;
    os[sp] = ok ? pr[sp * stride + d] : 0.f;
  }
  float m = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) m = fmaxf(m, ms[sp]);
  float l = 0.f, o = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    if (ms[sp] == -INFINITY) continue;  // a split that saw no block of this row
    const float w = exp2f(ms[sp] - m);
    l += ls[sp] * w;
    o += os[sp] * w;
  }
  out[row * kD + d] = static_cast<uint16_t>(f32_to_bf16_bits(o / l));
  if (lse && d == 0) lse[row] = (m + log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Compressed-attention branch (skill page, Step 2, compressed_attention, made
// causal like block scoring): the query at position i attends the compressed
// keys of the nv = floor((i+1)/64) blocks that end at or before it and takes
// the softmax-weighted sum of their compressed values.  A KV head's
// compressed keys (values) are NB rows of 128 dims; 64 of them side by side
// have the layout of one key block, so the sparse pipeline streams them
// unchanged: group e of this kernel is compressed rows 64e .. 64e+63, and a
// token attends rows 0 .. nv-1 (its "last visible key" is nv - 1).  Same
// work unit as the sparse forward: 16 tokens x one KV head, one token per
// wave, the G heads of the group in the MFMA columns.
// Epilogue: out = w_cmp * O_cmp, plus w_sparse * o_sparse when o_sparse is
// given (the weighted mix of pattern outputs of skill page Step 3, with given
// coefficients).  out may be o_sparse itself: each lane reads its four
// values of a row before it writes them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWin * 64, 1) void compressed_attn_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ kc,
                                                                       const uint16_t* __restrict__ vc,
                                                                       const uint16_t* o_sparse, uint16_t* out,
                                                                       float* __restrict__ lse, AttnShape s,
                                                                       float w_sparse, float w_cmp) {
  constexpr int kWaves = kWin;  // one token per wave
  extern __shared__ __align__(1024) unsigned char smem[];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15, gq = lane >> 4;
  const int nwin = (s.S_q + kWin - 1) / kWin;
  int bg_i, win;
  if (!map_window(blockIdx.x, nwin, s.B * s.H_kv, bg_i, win)) return;
  const int g = bg_i % s.H_kv;
  const int b = bg_i / s.H_kv;
  const size_t bg = static_cast<size_t>(bg_i);
  const int r0 = win * kWin;
  const int r = r0 + wave;
  const int off = seq_keys(s, b) - s.S_q;    // query row r sits at key position off + r
  const int nq = min(kWin, s.S_q - r0);      // tokens of the window
  const int nv_max = (off + r0 + nq) / kBS;  // compressed rows the window's last token sees
  const int ngrp = (nv_max + kBS - 1) / kBS; // groups of 64 rows to stream
  const BlockSrc<false> src{kc + bg * s.NB * kD, vc + bg * s.NB * kD, nullptr, s.NB, 0, s.H_kv, b, g, s.NB};
  const float sl2 = s.scale_log2;

  SparseState st;
  {
    const bool valid = r < s.S_q && hl < s.G;
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q + r) * kD + gq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) st.qf[ks] = valid ? as_bf16x8(load16(qrow + ks * 32)) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) st.qf[ks] = settle(st.qf[ks]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
    st.lim = (off + r + 1) / kBS - 1;  // last visible compressed row (-1: none)
  }
  // list entry e: group e | the window's tokens that see its first row
  // (token t sees row 64e iff off + r0 + t + 1 >= 64 (64e + 1))
  auto entry_at = [&](int e) -> uint32_t { return cmp_entry(e, off, r0, nq); };
  const SparseLane spl = sparse_lane(hl, gq);
  stream_pairs<kWaves>(smem, src, 0, ngrp, entry_at, wave, lane,
                       [&](const unsigned char* const* stg, const int* js, uint32_t cur0, uint32_t cur1) {
    const uint32_t bit = 1u << (16 + wave);
    attend_pair(st, spl, stg, js, (cur0 & bit) != 0u, (cur1 & bit) != 0u, lane, sl2);
  });

  const float l = sum_xor32(sum_xor16(st.l));
  if (r >= s.S_q || hl >= s.G) return;
  const int h = g * s.G + hl;
  const size_t row = static_cast<size_t>(b * s.H_q + h) * s.S_q + r;
  const float scl = l > 0.f ? w_cmp / l : 0.f;  // a token that sees no block: the branch is zero
  uint16_t* orow = out + row * kD + 4 * gq;
  const uint16_t* srow = o_sparse ? o_sparse + row * kD + 4 * gq : nullptr;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = st.o[dt][e] * scl;
    if (srow) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(srow + 16 * dt);
      y[0] = fmaf(w_sparse, bf16_lo(x[0]), y[0]);
      y[1] = fmaf(w_sparse, bf16_hi(x[0]), y[1]);
      y[2] = fmaf(w_sparse, bf16_lo(x[1]), y[2]);
      y[3] = fmaf(w_sparse, bf16_hi(x[1]), y[3]);
    }
    *reinterpret_cast<u32x2*>(orow + 16 * dt) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  }
  if (lse && gq == 0) lse[row] = l > 0.f ? (st.m + log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_compressed_attn(const uint16_t* q, const uint16_t* k_cmp, const uint16_t* v_cmp,
                                  const uint16_t* o_sparse, uint16_t* out, float* lse, const AttnShape& s,
                                  float w_sparse, float w_cmp, hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  const int nwin = (s.S_q + kWin - 1) / kWin;
  hipLaunchKernelGGL(compressed_attn_kernel, dim3(padded_grid(nwin, s.B * s.H_kv)), dim3(kWin * 64),
                     kStages * kStageBytes, stream, q, k_cmp, v_cmp, o_sparse, out, lse, s, w_sparse, w_cmp);
  return hipGetLastError();
}

int sparse_splits(int B, int H_kv, int S_q, int topk) {
  const long long units = static_cast<long long>(B) * H_kv * ((S_q + kWin - 1) / kWin);
  if (units >= 128) return 1;
  // about one workgroup per CU (256 CUs): more splits only add a second round
  const int by_units = static_cast<int>(256 / units);
  const int by_blocks = max(1, (topk + 3) / 4);  // keep >= ~4 blocks per split
  return max(1, min(16, min(by_units, by_blocks)));
}

size_t attn_workspace_bytes(const AttnShape& s) {
  const int ns = sparse_splits(s.B, s.H_kv, s.S_q, s.topk);
  if (ns <= 1) return 0;
  return static_cast<size_t>(ns) * s.B * s.H_q * s.S_q * kPartFloats * sizeof(float);
}

static_assert(kStages * kStageBytes + sparse_list_bytes(kMaxSparseBlocks) <= 163840,
              "the ring and the largest union list fit in the 160 KB of LDS");

template <bool DENSE, bool MIX = false>
static hipError_t launch_window(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* blk_idx,
                                uint16_t* out, float* lse, float* part, const AttnShape& s, hipStream_t stream,
                                MixArgs mx = MixArgs{nullptr, nullptr, 0.f, 0.f}) {
  const int nwin = (s.S_q + kWin - 1) / kWin;
  const dim3 grid(padded_grid(nwin, s.B * s.H_kv), DENSE ? 1 : s.nsplit);
  const size_t lds = kStages * kStageBytes + (DENSE ? 0 : sparse_list_bytes(s.NB));
  if constexpr (MIX) {
    hipLaunchKernelGGL((attn_window_kernel<false, false, true>), grid, dim3(Cfg<false>::kWaves * 64), lds, stream, q,
                       k, v, blk_idx, out, lse, part, s, mx);
    return hipGetLastError();
  }
  if constexpr (!DENSE) {  // the dense kernel has no paged form
    if (s.block_table) {
      hipLaunchKernelGGL((attn_window_kernel<false, true, false>), grid, dim3(Cfg<false>::kWaves * 64), lds, stream, q,
                         k, v, blk_idx, out, lse, part, s, mx);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_window_kernel<DENSE, false, false>), grid, dim3(Cfg<DENSE>::kWaves * 64), lds, stream, q,
                     k, v, blk_idx, out, lse, part, s, mx);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* blk_idx, uint16_t* out, float* lse,
                              const AttnShape& s_in, void* workspace, hipStream_t stream) {
  if (s_in.B == 0 || s_in.S_q == 0) return hipSuccess;
  AttnShape s = s_in;
  s.nsplit = sparse_splits(s.B, s.H_kv, s.S_q, s.topk);
  float* part = s.nsplit > 1 ? static_cast<float*>(workspace) : nullptr;
  hipError_t err = launch_window<false>(q, k, v, blk_idx, out, lse, part, s, stream);
  if (err != hipSuccess || s.nsplit == 1) return err;
  return launch_combine_splits(part, out, lse, s, stream);
}

hipError_t launch_combine_splits(const float* part, uint16_t* out, float* lse, const AttnShape& s,
                                 hipStream_t stream) {
  const size_t rows = static_cast<size_t>(s.B) * s.H_q * s.S_q;
  hipLaunchKernelGGL(combine_splits_kernel, dim3(rows), dim3(128), 0, stream, part, out, lse, s.nsplit, rows);
  return hipGetLastError();
}

hipError_t launch_mixed_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* blk_idx,
                             const uint16_t* k_cmp, const uint16_t* v_cmp, uint16_t* out, float* lse,
                             const AttnShape& s_in, float w_sparse, float w_cmp, void* workspace, hipStream_t stream) {
  if (s_in.B == 0 || s_in.S_q == 0) return hipSuccess;
  AttnShape s = s_in;
  s.nsplit = sparse_splits(s.B, s.H_kv, s.S_q, s.topk);
  if (s.nsplit > 1) {  // few query windows: the sparse output, then the branch mixed into it in place
    hipError_t err = launch_sparse_attn(q, k, v, blk_idx, out, lse, s_in, workspace, stream);
    if (err != hipSuccess) return err;
    return launch_compressed_attn(q, k_cmp, v_cmp, out, out, nullptr, s_in, w_sparse, w_cmp, stream);
  }
  return launch_window<false, true>(q, k, v, blk_idx, out, lse, nullptr, s, stream,
                                    MixArgs{k_cmp, v_cmp, w_sparse, w_cmp});
}

hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, const AttnShape& s_in, void*, hipStream_t stream) {
  if (s_in.B == 0 || s_in.S_q == 0) return hipSuccess;
  AttnShape s = s_in;
  s.nsplit = 1;
  return launch_window<true>(q, k, v, nullptr, out, lse, nullptr, s, stream);
}

}  // namespace infv2
