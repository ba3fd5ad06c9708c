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
constexpr float kRescaleSlack = 8.f;              // log2 units the running max may lag behind



// ---------------------------------------------------------------------------
// Sparse: 16x16x32 MFMAs, one token per 16-column block (lane = head hl,
// key quad gq).  MASK says which of the wave's tokens attend block j.
// ---------------------------------------------------------------------------
struct SparseState {
  bf16x8 qf[4];        // Q^T B operands, k-steps of 32 dims
  floatx4 o[8];        // O^T accumulators, 8 tiles of 16 dims
  float m, l;
  int lim;             // last visible key position of the token
};

// One online-softmax step of the wave's token over N attended blocks (N * 64
// keys): S^T = K Q^T for each block, one joint max / rescale, P, then
// O^T += V^T P^T.  Stage n holds block js[n].
template <int N>
__device__ __forceinline__ void sparse_step(SparseState& st, const SparseLane& ln, const unsigned char* const* stg,
                                            const int* js, float sl2, int gq) {
  // k-step outer, key tile inner: each step is 4 independent MFMAs whose K
  // fragments were all requested together
  floatx4 sacc[N][4];
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 kf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kf[kt] = as_bf16x8(load16(stg[n] + ln.k(ks) + kt * 16 * kRowBytes));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        sacc[n][kt] = mfma_16x16x32(kf[kt], st.qf[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : sacc[n][kt]);
    }
  // lane (hl, gq) holds keys 16*kt + 4*gq + e2 of head hl in each block
  float mx = -INFINITY;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    if (js[n] * kBS + kBS - 1 > st.lim) {  // wave-uniform: the block reaches past the token
      const int first = st.lim - js[n] * kBS - 4 * gq;  // keys 16*kt + e2 > first are masked
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          if (16 * kt + e2 > first) sacc[n][kt][e2] = -INFINITY;
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[n][kt][0], sacc[n][kt][1]), fmaxf(sacc[n][kt][2], sacc[n][kt][3])));
  }
  mx = max_xor32(max_xor16(mx)) * sl2;
  const bool grow = mx > st.m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mn = grow ? mx : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);  // m = -inf on a row's first block: 0
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
    st.m = mn;
  }
  const float nm = -st.m;
  bf16x8 pf[N][2];
  float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    uint32_t pw[8];
#pragma unroll
    for (int c2 = 0; c2 < 8; ++c2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[n][c2 >> 1][(c2 & 1) * 2], sl2, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[n][c2 >> 1][(c2 & 1) * 2 + 1], sl2, nm));
      pw[c2] = pack_bf16x2(p0, p1);
      rs0 += p0;
      rs1 += p1;
    }
    // k-step s2 of PV takes S^T tiles 2*s2 (slots 0..3) and 2*s2+1 (slots 4..7)
    pf[n][0] = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
    pf[n][1] = as_bf16x8(u32x4{pw[4], pw[5], pw[6], pw[7]});
  }
  st.l += rs0 + rs1;
  // O^T += V^T P^T.  The V^T operand of lane (hl, gq) for k-step s2 is keys
  // 32*s2 + 4*gq + {0..3} and 32*s2 + 16 + 4*gq + {0..3} of dim 16*dt + hl.
  // k-step outer, dim tiles inner in groups of 4: independent MFMAs.
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d0 = 0; d0 < 8; d0 += 4) {
        bf16x8 vf[4];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          const unsigned char* p = stg[n] + kTileBytes + ln.v(d0 + dd) + s2 * 32 * kRowBytes;
          vf[dd] = __builtin_shufflevector(lds_read_tr(p), lds_read_tr(p + 16 * kRowBytes), 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) st.o[d0 + dd] = mfma_16x16x32(vf[dd], pf[n][s2], st.o[d0 + dd]);
      }
}

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

template <bool DENSE>
__global__ __launch_bounds__(Cfg<DENSE>::kWaves * 64, 1) void attn_window_kernel(const uint16_t* __restrict__ q,
                                                                     const uint16_t* __restrict__ k,
                                                                     const uint16_t* __restrict__ v,
                                                                     const int32_t* __restrict__ blk_idx,
                                                                     uint16_t* __restrict__ out,
                                                                     float* __restrict__ lse,
                                                                     float* __restrict__ part, AttnShape s) {
  constexpr int kWaves = Cfg<DENSE>::kWaves;
  constexpr int T = Cfg<DENSE>::kTok;
  constexpr int NT = kWaves * 64;
  extern __shared__ __align__(1024) unsigned char smem[];
  uint32_t* bmask = reinterpret_cast<uint32_t*>(smem + kStages * kStageBytes);  // [NB], sparse only
  int* blist = reinterpret_cast<int*>(bmask + s.NB);                           // [NB], sparse only
  __shared__ int n_list;

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
  const int off = s.S_k - s.S_q;
  const int i_last = off + min(r0 + kWin, s.S_q) - 1;
  const int qb_last = i_last / kBS;
  const uint16_t* kg = k + bg * s.S_k * kD;
  const uint16_t* vg = v + bg * s.S_k * kD;
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
    dn.lim = s.causal ? min(off + r, s.S_k - 1) : s.S_k - 1;
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
      sp[t].lim = min(off + rw + t, s.S_k - 1);
    }
  }

  // ---- the union of attended blocks ---------------------------------------
  // Sparse: list entry = block index | (16-bit member mask of the window's
  // tokens) << 16, ascending by block.
  int nblk;
  if constexpr (DENSE) {
    nblk = s.causal ? qb_last + 1 : s.NB;
  } else {
    nblk = build_union_list<NT>(bmask, blist, &n_list, blk_idx, bg, r0, off, qb_last, s, wave, lane);
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
      if (e < nblk) stage_block(ring + e * kStageBytes, kg, vg, e, s.S_k, dl, wave, lane);
    // this wave's two tokens' visibility limits (a token past the end of the
    // queries takes its partner's)
    const int lim0 = s.causal ? min(off + rw, s.S_k - 1) : s.S_k - 1;
    const int lim1 = rw + 1 < s.S_q ? (s.causal ? min(off + rw + 1, s.S_k - 1) : s.S_k - 1) : lim0;
    const DenseLane dnl = dense_lane(lane);
    for (int j = 0; j < nblk; ++j) {
      wait_dma<kDma>(min(kStages - 2, nblk - 1 - j));
      __syncthreads();  // block j is in LDS; every wave is done with block j - 1
      if (j + kStages - 1 < nblk)
        stage_block(ring + ((j + kStages - 1) % kStages) * kStageBytes, kg, vg, j + kStages - 1, s.S_k, dl, wave,
                    lane);
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
    stream_pairs<kWaves>(smem, kg, vg, s.S_k, e_lo, e_hi, entry_at, wave, lane,
                         [&](const unsigned char* const* stg, const int* js, uint32_t cur0, uint32_t cur1) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t bit = 1u << (16 + wave * T + t);
        const bool m0 = (cur0 & bit) != 0u, m1 = (cur1 & bit) != 0u;   // cur1 = 0 past the list
        if (m0 && m1) sparse_step<2>(sp[t], spl, stg, js, sl2, lane >> 4);
        else if (m0) sparse_step<1>(sp[t], spl, stg, js, sl2, lane >> 4);
        else if (m1) sparse_step<1>(sp[t], spl, stg + 1, js + 1, sl2, lane >> 4);
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
      const float inv = 1.f / l;
      uint16_t* orow = out + (static_cast<size_t>(b * s.H_q + h) * s.S_q + r) * kD + 4 * gq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x2 w = {pack_bf16x2(sp[t].o[dt][0] * inv, sp[t].o[dt][1] * inv),
                         pack_bf16x2(sp[t].o[dt][2] * inv, sp[t].o[dt][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * dt) = w;
      }
      if (lse && gq == 0) lse[static_cast<size_t>(b * s.H_q + h) * s.S_q + r] = (sp[t].m + log2f(l)) * kLn2;
    }
  }
}

// Merge the split partials of each query row: m = max_s m_s,
// l = sum_s l_s 2^(m_s - m), O = sum_s o_s 2^(m_s - m) / l.  One workgroup of
// 128 threads (one per dim) per row.
__global__ __launch_bounds__(128) void combine_splits_kernel(const float* __restrict__ part,
                                                             uint16_t* __restrict__ out, float* __restrict__ lse,
                                                             int nsplit, size_t rows) {
  const size_t row = blockIdx.x;
  const int d = threadIdx.x;
  const size_t stride = rows * kPartFloats;
  float m = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, part[sp * stride + row * kPartFloats + 128]);
  float l = 0.f, o = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* pr = part + sp * stride + row * kPartFloats;
    const float ms = pr[128];
    if (ms == -INFINITY) continue;  // a split that saw no block of this row
    const float w = exp2f(ms - m);
    l += pr[129] * w;
    o += pr[d] * w;
  }
  out[row * kD + d] = static_cast<uint16_t>(f32_to_bf16_bits(o / l));
  if (lse && d == 0) lse[row] = (m + log2f(l)) * kLn2;
}

int sparse_splits(int B, int H_kv, int S_q, int topk) {
  const long long units = static_cast<long long>(B) * H_kv * ((S_q + kWin - 1) / kWin);
  if (units >= 128) return 1;
  const int by_units = static_cast<int>(512 / units);
  const int by_blocks = max(1, (topk + 3) / 4);  // keep >= ~4 blocks per split
  return max(1, min(16, min(by_units, by_blocks)));
}

size_t attn_workspace_bytes(const AttnShape& s) {
  const int ns = sparse_splits(s.B, s.H_kv, s.S_q, s.topk);
  if (ns <= 1) return 0;
  return static_cast<size_t>(ns) * s.B * s.H_q * s.S_q * kPartFloats * sizeof(float);
}

template <bool DENSE>
static hipError_t launch_window(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* blk_idx,
                                uint16_t* out, float* lse, float* part, const AttnShape& s, hipStream_t stream) {
  const int nwin = (s.S_q + kWin - 1) / kWin;
  const dim3 grid(padded_grid(nwin, s.B * s.H_kv), DENSE ? 1 : s.nsplit);
  const size_t lds = kStages * kStageBytes + (DENSE ? 0 : 2 * sizeof(int) * static_cast<size_t>(s.NB));
  hipLaunchKernelGGL((attn_window_kernel<DENSE>), grid, dim3(Cfg<DENSE>::kWaves * 64), lds, stream, q, k, v,
                     blk_idx, out, lse, part, s);
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
  const size_t rows = static_cast<size_t>(s.B) * s.H_q * s.S_q;
  hipLaunchKernelGGL(combine_splits_kernel, dim3(rows), dim3(128), 0, stream, part, out, lse, s.nsplit, rows);
  return hipGetLastError();
}

hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, const AttnShape& s_in, void*, hipStream_t stream) {
  if (s_in.B == 0 || s_in.S_q == 0) return hipSuccess;
  AttnShape s = s_in;
  s.nsplit = 1;
  return launch_window<true>(q, k, v, nullptr, out, lse, nullptr, s, stream);
}

}  // namespace infv2
