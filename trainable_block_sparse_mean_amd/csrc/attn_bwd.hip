// Backward of the block-sparse attention for gfx950 (dq, dk, dv).
//
// The attention is trained by back-propagation (skill page "Infllm V2 Dense
// Sparse Switchable Attention", Step 5: Training and Fine-tuning Procedure).
// The attended key set of each query is the forward's (initial blocks, causal
// block window, selected blocks); the selection itself carries no gradient.
// With P the softmax weights (recomputed from the forward's log-sum-exp),
// dP = dO V^T, D = <dO, O> per (token, head) and dS = P (dP - D):
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO,
// dK and dV summed over every (token, head of the group) that attends a key.
//
// Three kernels, in stream order:
//   1. bitmap: one bit per (KV head, block j, query token r) for the selected
//      entries of blk_idx that are not forced blocks of r (forced blocks are
//      recognised arithmetically).  Built per 32-token word in LDS, so every
//      bitmap word is written once and the result does not depend on order.
//   2. attn_bwd_dq_kernel, window-major like the forward (one workgroup = one
//      KV head x 16 query tokens, one token per wave, the window's union of
//      blocks streamed through the LDS ring in pairs).  Per member block:
//      S^T = K Q^T, P, dP^T = V dO^T (V's rows read like K's), dS, and
//      dQ^T += K^T dS^T (K's columns read with the transposing LDS read, as
//      the forward reads V^T).  It also writes D for kernel 3.
//   3. attn_bwd_dkdv_kernel, block-major: one workgroup = one KV head x one
//      64-key block, 4 waves of 16 keys.  It walks the tokens that attend the
//      block in pairs (32 (token, head) rows = the k-dimension of one
//      16x16x32 MFMA): S = Q K^T and dP = dO V^T with this wave's K and V
//      held in registers, then dV^T += dO^T P and dK^T += Q^T dS, where Q^T
//      and dO^T come from the pair's Q and dO rows in LDS through the
//      transposing read and P, dS are already laid out as the B operand.
//      Every key of the block is written once, so no atomics are needed.
#include "attn_common.hpp"

namespace infv2 {

constexpr int kBwdDqWaves = 16;        // dq kernel: one token per wave
constexpr int kBwdKvWaves = 4;         // dk/dv kernel: 16 keys per wave
constexpr int kPairRows = 32;          // (token, head) rows of a token pair
constexpr int kPairBytes = kPairRows * kRowBytes;  // Q (or dO) rows of a pair in LDS
constexpr int kMemberChunk = 1024;     // tokens scanned per member-list chunk

__host__ __device__ constexpr int bitmap_words(int S_q) { return (S_q + 31) / 32; }

// ---------------------------------------------------------------------------
// 1. selected-entry bitmap
// ---------------------------------------------------------------------------
__global__ void bwd_bitmap_zero_kernel(uint32_t* __restrict__ bm, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    bm[i] = 0u;
}

// One workgroup per (b, g, 32-token word): the word's bits of every key
// block are set in LDS (LDS atomics), then every bitmap word of the column is
// written once, so the bitmap needs no clearing and no global atomics.
constexpr int kBitmapThreads = 256;
__global__ __launch_bounds__(kBitmapThreads) void bwd_bitmap_build_kernel(const int32_t* __restrict__ blk_idx,
                                                                           uint32_t* __restrict__ bm, AttnShape s) {
  extern __shared__ uint32_t bits[];  // [NB]
  const size_t bg = blockIdx.y;
  const int word = blockIdx.x;
  const int r0 = word * 32;
  const int W = bitmap_words(s.S_q);
  const int off = s.S_k - s.S_q;
  for (int j = threadIdx.x; j < s.NB; j += kBitmapThreads) bits[j] = 0u;
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * s.topk; e += kBitmapThreads) {
    const int t = e / s.topk;
    const int r = r0 + t;
    if (r >= s.S_q) continue;
    const int j = blk_idx[(bg * s.S_q + r) * s.topk + (e - t * s.topk)];
    const int qb = (off + r) / kBS;
    // forced blocks of r (initial or window) are recognised by the dK/dV kernel itself
    if (j < s.n_init || j > qb - s.n_local) continue;  // also drops j < 0 and j > qb
    atomicOr(&bits[j], 1u << t);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < s.NB; j += kBitmapThreads) bm[(bg * s.NB + j) * W + word] = bits[j];
}

// ---------------------------------------------------------------------------
// 2. dq (and D)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdDqWaves * 64, 1) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ out, const float* __restrict__ lse, const uint16_t* __restrict__ dout,
    const int32_t* __restrict__ blk_idx, uint16_t* __restrict__ dq, float* __restrict__ dsum, AttnShape s,
    float scale) {
  constexpr int NT = kBwdDqWaves * 64;
  extern __shared__ __align__(1024) unsigned char smem[];
  uint32_t* bmask = reinterpret_cast<uint32_t*>(smem + kStages * kStageBytes);  // [NB]
  int* blist = reinterpret_cast<int*>(bmask + s.NB);                           // [NB]
  int* n_list = blist + s.NB;                                                  // list length

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15, gq = lane >> 4;
  const int nwin = (s.S_q + kWin - 1) / kWin;
  int bg_i, win;
  if (!map_window(blockIdx.x, nwin, s.B * s.H_kv, bg_i, win)) return;  // whole workgroup
  const int g = bg_i % s.H_kv;
  const int b = bg_i / s.H_kv;
  const size_t bg = static_cast<size_t>(bg_i);
  const int r0 = win * kWin;
  const int r = r0 + wave;
  const int off = s.S_k - s.S_q;
  const int qb_last = (off + min(r0 + kWin, s.S_q) - 1) / kBS;
  const uint16_t* kg = k + bg * s.S_k * kD;
  const uint16_t* vg = v + bg * s.S_k * kD;
  const float sl2 = s.scale_log2;

  // per-token operands: lane (head hl, dims 8*gq + 32*ks .. +7)
  const bool valid = r < s.S_q && hl < s.G;
  const int h = g * s.G + hl;
  const size_t row = (static_cast<size_t>(b) * s.H_q + h) * s.S_q + r;
  bf16x8 qf[4], df[4];
  float dpart = 0.f;
  {
    const uint16_t* qrow = q + row * kD + gq * 8;
    const uint16_t* drow = dout + row * kD + gq * 8;
    const uint16_t* orow = out + row * kD + gq * 8;
    u32x4 oraw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[ks] = valid ? as_bf16x8(load16(qrow + ks * 32)) : bf16x8{};
      df[ks] = valid ? as_bf16x8(load16(drow + ks * 32)) : bf16x8{};
      oraw[ks] = valid ? load16(orow + ks * 32) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[ks] = settle(qf[ks]);
      df[ks] = settle(df[ks]);
      const u32x4 dw = as_u32x4(df[ks]);
      const u32x4 ow = as_u32x4(settle(as_bf16x8(oraw[ks])));
#pragma unroll
      for (int c = 0; c < 4; ++c)
        dpart += bf16_lo(dw[c]) * bf16_lo(ow[c]) + bf16_hi(dw[c]) * bf16_hi(ow[c]);
    }
  }
  // D = <dO, O> of head hl: the four row quads hold the 128 dims
  const float Dh = sum_xor32(sum_xor16(dpart));
  const float lse2 = valid ? lse[row] * kLog2e : 0.f;
  if (valid && gq == 0) dsum[row] = Dh;
  const int lim = min(off + r, s.S_k - 1);

  const int nblk = build_union_list<NT>(bmask, blist, n_list, blk_idx, bg, r0, off, qb_last, s, wave, lane);
  auto entry_at = [&](int e) -> uint32_t { return e < nblk ? static_cast<uint32_t>(blist[e]) : 0u; };

  const SparseLane ln = sparse_lane(hl, gq);
  floatx4 dqa[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dqa[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one member block: lane (hl, gq) holds keys 16*kt + 4*gq + e of head hl.
  // Two halves of 32 keys (key tiles 2*s2 and 2*s2+1): S^T and dP^T of the
  // half, dS, then k-step s2 of dQ^T += K^T dS^T, which takes exactly those
  // two tiles (slots 0..3 and 4..7).
  auto item = [&](const unsigned char* stg_ptr, int j) {
    const uint32_t stg = lds_addr(stg_ptr);           // the stage's LDS address, converted once
    const bool need_mask = j * kBS + kBS - 1 > lim;   // wave-uniform
    const int first = lim - j * kBS - 4 * gq;         // keys 16*kt + e > first are masked
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      floatx4 sacc[2], dpa[2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 kf[2], vf[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int kt = 2 * s2 + x;
          kf[x] = as_bf16x8(lds_load16_at(stg + ln.k(ks) + kt * 16 * kRowBytes));
          vf[x] = as_bf16x8(lds_load16_at(stg + kTileBytes + ln.k(ks) + kt * 16 * kRowBytes));
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          sacc[x] = mfma_16x16x32(kf[x], qf[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : sacc[x]);
          dpa[x] = mfma_16x16x32(vf[x], df[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : dpa[x]);
        }
      }
      // keys past the token (only in its own block): -inf scores, so p = 0.
      // A branch marked unlikely: otherwise the compiler tests every key of
      // every block.
      if (__builtin_expect(need_mask, 0)) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * (2 * s2 + x) + e > first) sacc[x][e] = -INFINITY;
      }
      uint32_t w[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int x = c >> 1, e0 = (c & 1) * 2;
        float d2[2];
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int e = e0 + y;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[x][e], sl2, -lse2));
          d2[y] = p * (dpa[x][e] - Dh);
        }
        w[c] = pack_bf16x2(d2[0], d2[1]);
      }
      const bf16x8 dsf = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
      // all eight K^T fragments in flight before the dQ products
      bf16x8 kt_f[8];
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const uint32_t p = stg + ln.v(dd) + s2 * 32 * kRowBytes;
        kt_f[dd] = __builtin_shufflevector(lds_read_tr_at(p), lds_read_tr_at(p + 16 * kRowBytes), 0, 1, 2, 3, 4, 5, 6,
                                           7);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) dqa[dd] = mfma_16x16x32(kt_f[dd], dsf, dqa[dd]);
    }
  };

  const uint32_t bit = 1u << (16 + wave);
  const BlockSrc<false> src{kg, vg, nullptr, s.NB, 0, s.H_kv, 0, 0, s.S_k};
  stream_pairs<kBwdDqWaves, true>(smem, src, 0, nblk, entry_at, wave, lane,
                            [&](const unsigned char* const* stg, const int* js, uint32_t cur0, uint32_t cur1) {
                              // one copy of the item code for both blocks of the pair
#pragma unroll 1
                              for (int n = 0; n < 2; ++n)
                                if (((n == 0 ? cur0 : cur1) & bit) != 0u) item(stg[n], js[n]);  // cur1 = 0 past the list
                            });

  if (valid) {
    uint16_t* grow = dq + row * kD + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x2 wv = {pack_bf16x2(dqa[dt][0] * scale, dqa[dt][1] * scale),
                        pack_bf16x2(dqa[dt][2] * scale, dqa[dt][3] * scale)};
      *reinterpret_cast<u32x2*>(grow + 16 * dt) = wv;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dk, dv
// ---------------------------------------------------------------------------
// LDS: a ring of kPairBufs buffers, each holding one token pair's Q rows,
// dO rows and the 32 rows' log-sum-exp and D (64 floats), then the member
// list of the current chunk (16-bit offsets from the chunk's first token)
// and its length: 51 KB, so that three workgroups (12 waves of at most 168
// VGPRs) share a CU.
constexpr int kPairBufs = 3;                                      // 2 pairs in flight
constexpr int kStatsBytes = 2 * kPairRows * 4;                    // lse[32], D[32]
constexpr int kKvBufBytes = 2 * kPairBytes + kStatsBytes;         // Q + dO + stats of one pair
constexpr int kKvLdsBytes = kPairBufs * kKvBufBytes + kMemberChunk * 2 + 16;
constexpr int kPairDma = 5;                                       // loads per wave per pair

// Issue the loads of one token pair into an LDS buffer: Q and dO rows (row
// 16*t + hd of a tile is head hd of token t) and the rows' log-sum-exp and D.
// Heads >= G and a missing second token re-read a valid row (their P and dS
// are zeroed).  Each wave issues kPairDma loads.
__device__ __forceinline__ void stage_pair(uint32_t buf_lds, const uint16_t* qg, const uint16_t* dg, const float* lg,
                                           const float* sg, int S_q, int G, int rA, int rB, int wave, int lane) {
  // 32 rows x 256 B per tile = 8 loads of 4 rows; each of the 4 waves moves 2
  const int sub = lane >> 4, slot = lane & 15;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int rw = (wave * 2 + n) * 4 + sub;          // row of the tile
    const int t = rw >> 4, hd = min(rw & 15, G - 1);
    const int tok = t == 0 ? rA : rB;
    const uint32_t voff = static_cast<uint32_t>((static_cast<size_t>(hd) * S_q + tok) * kRowBytes) +
                          static_cast<uint32_t>((slot ^ swz(rw)) << 4);
    const uint32_t lds = buf_lds + (wave * 2 + n) * 1024;
    dma16(qg, voff, lds);
    dma16(dg, voff, lds + kPairBytes);
  }
  // stats: wave 0 / 1 = lse of token A / B, wave 2 / 3 = D of token A / B
  const int tok = (wave & 1) ? rB : rA;
  const uint32_t soff = static_cast<uint32_t>((static_cast<size_t>(min(lane, G - 1)) * S_q + tok) * 4);
  if (lane < 16) dma4(wave < 2 ? lg : sg, soff, buf_lds + 2 * kPairBytes + wave * 64);
}

__global__ __launch_bounds__(kBwdKvWaves * 64, 3) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout, const float* __restrict__ dsum,
    const uint32_t* __restrict__ bm, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ part, AttnShape s, float scale) {
  extern __shared__ __align__(1024) unsigned char smem[];
  uint16_t* mlist = reinterpret_cast<uint16_t*>(smem + kPairBufs * kKvBufBytes);
  int* mcount = reinterpret_cast<int*>(mlist + kMemberChunk);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, gq = lane >> 4;
  // (KV head, piece, block): the workgroups that run together read the Q and
  // dO rows of one token range of one KV head (a working set the last-level
  // cache can hold), heaviest blocks first
  // With a multiple of 8 pieces, each XCD takes its own pieces (XCD x:
  // pieces x, x + 8, ...; the hardware deals workgroup n to XCD n % 8), so a
  // token's Q and dO rows are gathered into one XCD's L2 rather than into
  // every XCD that runs one of its blocks.  Every piece holds the same number
  // of (token, block) items, so the XCDs stay balanced.
  int j, piece;
  size_t bg;
  if (s.nsplit % kXcds == 0) {
    const int xcd = static_cast<int>(blockIdx.x % kXcds);
    const int kx = static_cast<int>(blockIdx.x / kXcds);
    const int per = s.nsplit / kXcds;  // pieces per XCD
    j = kx % s.NB;
    piece = ((kx / s.NB) % per) * kXcds + xcd;
    bg = static_cast<size_t>(kx / s.NB / per);
  } else {
    j = blockIdx.x % s.NB;
    piece = (blockIdx.x / s.NB) % s.nsplit;
    bg = blockIdx.x / s.NB / s.nsplit;
  }
  const int g = static_cast<int>(bg % s.H_kv);
  const int b = static_cast<int>(bg / s.H_kv);
  const int off = s.S_k - s.S_q;
  const float sl2 = s.scale_log2;
  const int W = bitmap_words(s.S_q);

  // this wave's 16 keys: key = 64*j + 16*wave + l16 (rows past S_k re-read
  // row S_k - 1; no query sees them)
  const int key = j * kBS + wave * 16 + l16;
  bf16x8 kf[4], vf[4];  // B operands: lane (key l16, dims 8*gq + 32*ks .. +7)
  {
    const size_t krow = (bg * s.S_k + min(key, s.S_k - 1)) * kD + gq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[ks] = settle(as_bf16x8(load16(k + krow + ks * 32)));
      vf[ks] = settle(as_bf16x8(load16(v + krow + ks * 32)));
    }
  }
  floatx4 dka[8], dva[8];  // dK^T, dV^T tiles: lane (key l16, dims 16*dt + 4*gq + e)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    dka[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    dva[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* qg = q + (static_cast<size_t>(b) * s.H_q + g * s.G) * s.S_q * kD;
  const uint16_t* dg = dout + (static_cast<size_t>(b) * s.H_q + g * s.G) * s.S_q * kD;
  const size_t hrow0 = (static_cast<size_t>(b) * s.H_q + g * s.G) * s.S_q;  // (head 0 of the group, token 0)
  const float* lg = lse + hrow0;
  const float* sg = dsum + hrow0;
  const uint32_t lbase = lds_addr(smem);
  // A-operand read offsets within a pair tile: lane (row l16 of a 16-row
  // tile, dims 8*gq + 32*ks); transposing reads: rows 4*gq + l16/4, dims
  // 16*dt + 4*(l16 % 4)
  const SparseLane ln = sparse_lane(l16, gq);

  // tokens that can see block j, and those for which it is a forced block
  const int r_first = max(0, j * kBS - off);
  const int f_hi = j < s.n_init ? s.S_q : min(s.S_q, (j + s.n_local) * kBS - off);
  const uint32_t* bmrow = bm + (bg * s.NB + j) * W;
  // this piece's tokens: [t_lo, t_hi), the same token range for every block
  // (whole bitmap words).  The chunks, and the pairs within a chunk, are
  // walked downwards from the top of the piece: on unrelated selections every
  // visible block has about the same share of member tokens at any position,
  // so the workgroups of a piece start at the same token and move down it at
  // about the same pace, and the Q and dO rows they gather are shared through
  // L2 instead of each being fetched once per block.
  const int share = ((s.S_q + s.nsplit - 1) / s.nsplit + 31) & ~31;
  const int t_lo = min(s.S_q, piece * share);
  const int t_hi = min(s.S_q, (piece + 1) * share);
  const int m_lo = max(r_first, t_lo);  // first token that can be a member
  const int nchunk = t_hi > m_lo ? (t_hi - t_lo + kMemberChunk - 1) / kMemberChunk : 0;

  for (int ci = nchunk - 1; ci >= 0; --ci) {
    const int c0 = t_lo + ci * kMemberChunk;
    if (c0 + kMemberChunk <= m_lo) break;  // this chunk and those below hold no member
    // member tokens of [c0, c0 + kMemberChunk), ascending, built by wave 0
    if (wave == 0) {
      const int r32 = c0 + 32 * lane;  // this lane's word (lanes 0..31)
      uint32_t bits = 0u;
      if (lane < kMemberChunk / 32 && r32 < t_hi) {
        bits = bmrow[r32 >> 5];
        // forced: [r_first, f_hi)
        const int lo = max(r_first - r32, 0), hi = min(f_hi - r32, 32);
        if (hi > lo) bits |= (hi - lo == 32 ? ~0u : ((1u << (hi - lo)) - 1u) << lo);
        // keep [m_lo, t_hi)
        if (r32 < m_lo) bits &= m_lo - r32 >= 32 ? 0u : ~((1u << (m_lo - r32)) - 1u);
        if (t_hi - r32 < 32) bits &= (1u << (t_hi - r32)) - 1u;
      }
      // exclusive prefix of popcounts over the 32 words
      const int cnt = __popc(bits);
      int pre = cnt;
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) {
        const int o = __shfl_up(pre, d, 64);
        if ((lane & 31) >= d) pre += o;
      }
      const int total = __shfl(pre, 31, 64);
      int pos = pre - cnt;
      while (bits) {
        const int bt = __builtin_ctz(bits);
        mlist[pos++] = static_cast<uint16_t>(r32 + bt - c0);
        bits &= bits - 1u;
      }
      if (lane == 0) *mcount = total;
    }
    __syncthreads();
    const int nm = *mcount;
    const int npair = (nm + 1) / 2;
    // the p-th pair walked is the (npair - 1 - p)-th of the ascending list
    auto pair_tok = [&](int p, int x) {
      const int pq = npair - 1 - p;
      return c0 + (2 * pq + x < nm ? mlist[2 * pq + x] : mlist[2 * pq]);
    };
    auto stage = [&](int p) {
      stage_pair(lbase + (p % kPairBufs) * kKvBufBytes, qg, dg, lg, sg, s.S_q, s.G, pair_tok(p, 0), pair_tok(p, 1),
                 wave, lane);
    };
#pragma unroll
    for (int x = 0; x < kPairBufs - 1; ++x)
      if (x < npair) stage(x);
    for (int p = 0; p < npair; ++p) {
      const int ahead = min(kPairBufs - 2, npair - 1 - p);  // later pairs whose loads are already issued
      if (ahead >= 2) wait_vmcnt<2 * kPairDma>();
      else if (ahead == 1) wait_vmcnt<kPairDma>();
      else wait_vmcnt<0>();
      __syncthreads();  // pair p is in LDS; every wave is done with pair p - 1
      if (p + kPairBufs - 1 < npair) stage(p + kPairBufs - 1);  // into pair p - 1's buffer
      const unsigned char* qt = smem + (p % kPairBufs) * kKvBufBytes;
      const unsigned char* dt_ = qt + kPairBytes;
      const float* st = reinterpret_cast<const float*>(qt + 2 * kPairBytes);  // lse[32], D[32]
      const int pq = npair - 1 - p;
      const int tA = c0 + mlist[2 * pq];
      const bool hasB = 2 * pq + 1 < nm;
      const int tB = hasB ? c0 + mlist[2 * pq + 1] : tA;
      // log-sum-exp (log2 units) and D of the rows this lane holds: (token t, heads 4*gq .. 4*gq+3)
      float lr[2][4], dr[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(st + 16 * t + 4 * gq);
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(st + 32 + 16 * t + 4 * gq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lr[t][e] = l4[e] * kLog2e;
          dr[t][e] = d4[e];
        }
      }
      // S = Q K^T and dP = dO V^T for the pair: tile t = token t's 16 heads
      floatx4 sacc[2], dpa[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
        dpa[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 qa = as_bf16x8(load16(qt + t * 16 * kRowBytes + ln.k(ks)));
          const bf16x8 da = as_bf16x8(load16(dt_ + t * 16 * kRowBytes + ln.k(ks)));
          sacc[t] = mfma_16x16x32(qa, kf[ks], sacc[t]);
          dpa[t] = mfma_16x16x32(da, vf[ks], dpa[t]);
        }
      }
      // rows of the result: (token t, head 4*gq + e); column: this lane's key
      uint32_t pw[4], sw[4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int tok = t == 0 ? tA : tB;
        const bool tok_ok = t == 0 || hasB;
        const int i = off + tok;
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = tok_ok && 4 * gq + e < s.G && key <= i;
          const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sacc[t][e], sl2, -lr[t][e])) : 0.f;
          pv[e] = p;
          dsv[e] = p * (dpa[t][e] - dr[t][e]);
        }
        pw[2 * t] = pack_bf16x2(pv[0], pv[1]);
        pw[2 * t + 1] = pack_bf16x2(pv[2], pv[3]);
        sw[2 * t] = pack_bf16x2(dsv[0], dsv[1]);
        sw[2 * t + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      // B operands: k-slots 8*gq .. 8*gq+7 = (token A, heads 4gq..4gq+3), (token B, same heads)
      const bf16x8 pb = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
      const bf16x8 sb = as_bf16x8(u32x4{sw[0], sw[1], sw[2], sw[3]});
      // dV^T += dO^T P and dK^T += Q^T dS: A operands by transposing reads of
      // rows 4*gq .. 4*gq+3 of each token's tile, dims 16*dt .. 16*dt+15
#pragma unroll
      for (int d0 = 0; d0 < 8; d0 += 4) {
        bf16x8 oa[4], qa[4];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          const unsigned char* pq = qt + ln.v(d0 + dd);
          const unsigned char* pd = dt_ + ln.v(d0 + dd);
          oa[dd] = __builtin_shufflevector(lds_read_tr(pd), lds_read_tr(pd + 16 * kRowBytes), 0, 1, 2, 3, 4, 5, 6, 7);
          qa[dd] = __builtin_shufflevector(lds_read_tr(pq), lds_read_tr(pq + 16 * kRowBytes), 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          dva[d0 + dd] = mfma_16x16x32(oa[dd], pb, dva[d0 + dd]);
          dka[d0 + dd] = mfma_16x16x32(qa[dd], sb, dka[d0 + dd]);
        }
      }
    }
    __syncthreads();  // the member list and the ring are free for the next chunk
  }

  if (s.nsplit > 1) {
    // fp32 partial of this piece: [dK (64 keys x 128), dV (64 keys x 128)], unscaled
    float* pp = part + ((bg * s.NB + j) * s.nsplit + piece) * (2 * kBS * kD) + (wave * 16 + l16) * kD + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      *reinterpret_cast<floatx4*>(pp + 16 * dt) = dka[dt];
      *reinterpret_cast<floatx4*>(pp + kBS * kD + 16 * dt) = dva[dt];
    }
  } else if (key < s.S_k) {
    const size_t orow = (bg * s.S_k + key) * kD + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x2 wk = {pack_bf16x2(dka[dt][0] * scale, dka[dt][1] * scale),
                        pack_bf16x2(dka[dt][2] * scale, dka[dt][3] * scale)};
      const u32x2 wv = {pack_bf16x2(dva[dt][0], dva[dt][1]), pack_bf16x2(dva[dt][2], dva[dt][3])};
      *reinterpret_cast<u32x2*>(dk + orow + 16 * dt) = wk;
      *reinterpret_cast<u32x2*>(dv + orow + 16 * dt) = wv;
    }
  }
}

// Sum the pieces of each (KV head, block) in piece order and round to bf16.
// One workgroup of 256 threads per block; thread t handles dims 4*(t%32) of
// keys t/32 + 8*n.
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                              AttnShape s, float scale) {
  const int j = blockIdx.x % s.NB;
  const size_t bg = blockIdx.x / s.NB;
  const float* pb = part + (bg * s.NB + j) * s.nsplit * (2 * kBS * kD);
  const int d4 = (threadIdx.x & 31) * 4;
  for (int kr = threadIdx.x >> 5; kr < kBS; kr += 8) {
    const int key = j * kBS + kr;
    if (key >= s.S_k) break;
    floatx4 ak = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
    for (int pc = 0; pc < s.nsplit; ++pc) {
      const float* pp = pb + pc * (2 * kBS * kD) + kr * kD + d4;
      ak += *reinterpret_cast<const floatx4*>(pp);
      av += *reinterpret_cast<const floatx4*>(pp + kBS * kD);
    }
    const size_t orow = (bg * s.S_k + key) * kD + d4;
    *reinterpret_cast<u32x2*>(dk + orow) = u32x2{pack_bf16x2(ak[0] * scale, ak[1] * scale),
                                                 pack_bf16x2(ak[2] * scale, ak[3] * scale)};
    *reinterpret_cast<u32x2*>(dv + orow) = u32x2{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
  }
}

// pieces per key block: enough that the block every query attends (or the
// most selected ones) does not outlast the rest of the grid, and narrow token
// ranges, whose Q and dO rows the workgroups of a piece share through L2
// (16 pieces: dK/dV 9.34 -> 7.28 ms at 32k against 4, for 1.07 GB of partials)
int bwd_pieces(int S_q) { return S_q >= 3 * 4096 ? 16 : (S_q >= 4096 ? 2 : 1); }

// ---------------------------------------------------------------------------
size_t attn_bwd_workspace_bytes(const AttnShape& s) {
  const size_t dsum = (static_cast<size_t>(s.B) * s.H_q * s.S_q * sizeof(float) + 255) & ~static_cast<size_t>(255);
  const size_t bmw = static_cast<size_t>(s.B) * s.H_kv * s.NB * bitmap_words(s.S_q);
  const int np = bwd_pieces(s.S_q);
  const size_t parts = np > 1 ? static_cast<size_t>(s.B) * s.H_kv * s.NB * np * (2 * kBS * kD) * sizeof(float) : 0;
  return dsum + ((bmw * sizeof(uint32_t) + 255) & ~static_cast<size_t>(255)) + parts;
}

hipError_t launch_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                                  const float* lse, const uint16_t* dout, const int32_t* blk_idx, uint16_t* dq,
                                  uint16_t* dk, uint16_t* dv, const AttnShape& s, float scale, void* workspace,
                                  hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) {
    // no query: every key and value gradient is zero
    const size_t n = static_cast<size_t>(s.B) * s.H_kv * s.S_k * kD / 2;  // bf16 pairs as 32-bit words
    if (n > 0) {
      hipLaunchKernelGGL(bwd_bitmap_zero_kernel, dim3(256), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(dk), n);
      hipLaunchKernelGGL(bwd_bitmap_zero_kernel, dim3(256), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(dv), n);
    }
    return hipGetLastError();
  }
  float* dsum = static_cast<float*>(workspace);
  const size_t dsum_bytes = (static_cast<size_t>(s.B) * s.H_q * s.S_q * sizeof(float) + 255) & ~static_cast<size_t>(255);
  uint32_t* bm = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(workspace) + dsum_bytes);
  const size_t bmw = static_cast<size_t>(s.B) * s.H_kv * s.NB * bitmap_words(s.S_q);
  float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + dsum_bytes +
                                         ((bmw * sizeof(uint32_t) + 255) & ~static_cast<size_t>(255)));
  AttnShape sk = s;
  sk.nsplit = bwd_pieces(s.S_q);
  if (s.topk > 0)
    hipLaunchKernelGGL(bwd_bitmap_build_kernel, dim3(bitmap_words(s.S_q), s.B * s.H_kv), dim3(kBitmapThreads),
                       static_cast<size_t>(s.NB) * sizeof(uint32_t), stream, blk_idx, bm, s);
  else
    hipLaunchKernelGGL(bwd_bitmap_zero_kernel, dim3(1024), dim3(256), 0, stream, bm, bmw);
  const int nwin = (s.S_q + kWin - 1) / kWin;
  const size_t dq_lds = kStages * kStageBytes + sparse_list_bytes(s.NB);
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3(padded_grid(nwin, s.B * s.H_kv)), dim3(kBwdDqWaves * 64), dq_lds,
                     stream, q, k, v, out, lse, dout, blk_idx, dq, dsum, s, scale);
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3(s.B * s.H_kv * s.NB * sk.nsplit), dim3(kBwdKvWaves * 64), kKvLdsBytes,
                     stream, q, k, v, lse, dout, dsum, bm, dk, dv, part, sk, scale);
  if (sk.nsplit > 1)
    hipLaunchKernelGGL(bwd_dkdv_reduce_kernel, dim3(s.B * s.H_kv * s.NB), dim3(256), 0, stream, part, dk, dv, sk,
                       scale);
  return hipGetLastError();
}

}  // namespace infv2
