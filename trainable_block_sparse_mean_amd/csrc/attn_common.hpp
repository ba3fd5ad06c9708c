// Shared pieces of the gfx950 attention kernels (forward and backward):
// the LDS layout of a K/V block, the direct-to-LDS staging of blocks into a
// ring, the XCD-aware window mapping, the per-window union of attended blocks
// and the loop that streams that union through the ring in pairs.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kWin = 16;                          // tokens per workgroup
constexpr int kRowBytes = kD * 2;                 // one K or V row in LDS
constexpr int kTileBytes = kBS * kRowBytes;       // one 64-key block of K (or V)
constexpr int kStageBytes = 2 * kTileBytes;       // K + V of one block
constexpr int kStages = 4;                        // LDS ring: 3 blocks in flight
constexpr int kXcds = 8;                          // workgroups are dealt round-robin to 8 XCDs
constexpr int kXcdGroup = 4;                      // adjacent windows kept together on one XCD

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Reads at a 32-bit LDS address.  Where a stage pointer is picked at run time
// the compiler cannot trace it back to shared memory: plain reads of it become
// flat loads (which also count against vmcnt, so every wait for them would
// wait for the ring's direct-to-LDS loads in flight too), and even LDS-typed
// reads of it rebuild and null-check the 64-bit generic address each time.
// Converting the stage pointer once (lds_addr) and reading at offsets from it
// avoids both.
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
__device__ __forceinline__ u32x4 lds_load16_at(uint32_t a) { return *(const lds_u32x4*)(a); }
__device__ __forceinline__ bf16x4 lds_read_tr_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a));
}

__device__ __forceinline__ floatx16 mfma_32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


// Wait until at most `in_flight` later blocks' loads of this wave are
// pending; each block is `per_block` loads per wave.
template <int per_block>
__device__ __forceinline__ void wait_dma(int in_flight) {
  static_assert(per_block == 2 || per_block == 4, "vmcnt immediates below");
  if (in_flight >= 2) {
    if constexpr (per_block == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  } else if (in_flight == 1) {
    if constexpr (per_block == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// Per-lane byte offsets, within a 64-key block, of the 16-byte chunks this
// lane moves.  A tile (K or V of one block) is 16 chunks of 4 rows (1 KB =
// 64 lanes x 16 B per load); each of the WAVES waves moves 16 / WAVES of
// them for K and as many for V.  A full block needs no clamping; in a
// partial last block, rows past S_k - 1 re-read row S_k - 1 (finite, masked).
template <int WAVES>
struct DmaLane {
  static constexpr int kChunks = 16 / WAVES;
  uint32_t off[kChunks];
};
// The lane id, read in asm so that it is recomputed where it is used rather
// than kept live (and possibly spilled) across a loop.
__device__ __forceinline__ int lane_id_opaque() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

template <int WAVES>
__device__ __forceinline__ DmaLane<WAVES> dma_lane(int wave, int lane) {
  DmaLane<WAVES> d;
  const int sub = lane >> 4, slot = lane & 15;
#pragma unroll
  for (int n = 0; n < DmaLane<WAVES>::kChunks; ++n) {
    const int row = (wave * DmaLane<WAVES>::kChunks + n) * 4 + sub;
    d.off[n] = static_cast<uint32_t>(row * kRowBytes + ((slot ^ swz(row)) << 4));
  }
  return d;
}

// Issue the loads of one key block into one stage of the ring: kb and vb
// point at the block's first K and V rows, nrows (1..64) of which hold
// keys.  Rows past the last key re-read that key's row (finite, masked).
template <int WAVES>
__device__ __forceinline__ void stage_block(uint32_t stage_lds, const uint16_t* kb16, const uint16_t* vb16, int nrows,
                                            const DmaLane<WAVES>& d, int wave, int lane) {
  constexpr int C = DmaLane<WAVES>::kChunks;
  const char* kb = reinterpret_cast<const char*>(kb16);
  const char* vb = reinterpret_cast<const char*>(vb16);
  if (nrows >= kBS) {
#pragma unroll
    for (int n = 0; n < C; ++n) {
      const uint32_t lds = stage_lds + (wave * C + n) * 1024;
      dma16(kb, d.off[n], lds);
      dma16(vb, d.off[n], lds + kTileBytes);
    }
  } else {
    const int sub = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int n = 0; n < C; ++n) {
      const int row = (wave * C + n) * 4 + sub;
      const int crow = min(row, nrows - 1);
      const uint32_t off = static_cast<uint32_t>(crow * kRowBytes + ((slot ^ swz(row)) << 4));
      const uint32_t lds = stage_lds + (wave * C + n) * 1024;
      dma16(kb, off, lds);
      dma16(vb, off, lds + kTileBytes);
    }
  }
}

// Where a KV head's blocks live: PAGED = false, the contiguous [S_k][D] rows
// of one (batch, KV head) at k / v; PAGED = true, pages of a paged cache based
// at k / v, found through the block table (page ids clamped into range, so a
// bad table cannot address past the pages).  krows(j) / vrows(j) give block
// j's first row, keys(j) how many of its rows hold keys.  The contiguous form
// is a separate instantiation so that prefill carries none of the paging.
template <bool PAGED>
struct BlockSrc {
  const uint16_t* k;
  const uint16_t* v;
  const int* table;  // PAGED only
  int nb, num_pages, H_kv, b, g, S_k;
  __device__ __forceinline__ size_t rows(int j) const {
    if constexpr (!PAGED) {
      return static_cast<size_t>(j) * kBS * kD;
    } else {
      // read through the constant address space: the index is wave-uniform,
      // so this is a scalar load (counted by lgkmcnt).  A vector load here
      // would be counted by vmcnt, and waiting for it would also wait for the
      // direct-to-LDS loads just issued for the previous block.
      typedef __attribute__((address_space(4))) const int const_int;
      const int page = min(max(((const_int*)(table))[static_cast<size_t>(b) * nb + j], 0), num_pages - 1);
      return (static_cast<size_t>(page) * H_kv + g) * kBS * kD;
    }
  }
  __device__ __forceinline__ const uint16_t* krows(int j) const { return k + rows(j); }
  __device__ __forceinline__ const uint16_t* vrows(int j) const { return v + rows(j); }
  __device__ __forceinline__ int keys(int j) const { return min(kBS, S_k - j * kBS); }
};

template <int WAVES, typename Src>
__device__ __forceinline__ void stage_src(uint32_t stage_lds, const Src& src, int j, const DmaLane<WAVES>& d,
                                          int wave, int lane) {
  stage_block<WAVES>(stage_lds, src.krows(j), src.vrows(j), src.keys(j), d, wave, lane);
}

// Workgroup -> (KV head, window).  The hardware deals workgroups to the XCDs
// round-robin; this maps the k-th workgroup of every XCD so that each XCD
// runs groups of `gs` (<= kXcdGroup) adjacent windows of one KV head
// together (they stream the same K/V blocks through that XCD's L2), latest
// (heaviest) windows first.  Returns false for padding workgroups.
__host__ __device__ constexpr int xcd_group(int nwin) { return nwin < kXcdGroup ? nwin : kXcdGroup; }

__device__ __forceinline__ bool map_window(int n, int nwin, int nheads, int& head, int& win) {
  const int gs = xcd_group(nwin);
  const int xcd = n % kXcds, k = n / kXcds;
  const int rank = (k / gs) * kXcds + xcd;  // index of a group of gs windows
  const int ngrp = (nwin + gs - 1) / gs;
  head = rank % nheads;
  const int grp = ngrp - 1 - rank / nheads;
  win = grp * gs + (k % gs);
  return grp >= 0 && win < nwin;
}

__host__ __device__ constexpr int padded_grid(int nwin, int nheads) {
  // ranks needed: ngrp * nheads, rounded up to whole rounds of kXcds
  return ((((nwin + xcd_group(nwin) - 1) / xcd_group(nwin)) * nheads + kXcds - 1) / kXcds) * kXcds *
         xcd_group(nwin);
}

// Per-lane LDS byte offsets of the sparse fragment reads within a stage:
// K (A operand of S^T = K Q^T) for k-step ks at row hl (+16 rows per key
// tile), and V (transposing reads, A operand of O^T += V^T P^T) for dim tile
// dt at row 4*gq + hl/4 (+16 rows per half, +32 per k-step).  The swizzle
// is an XOR, so the offsets for k-step ks (dim tile dt) are the ks = 0
// (dt = 0) offset XOR ks << 6 (dt << 5): one register each.
struct SparseLane {
  uint32_t k0, v0;
  __device__ __forceinline__ uint32_t k(int ks) const { return k0 ^ static_cast<uint32_t>(ks << 6); }
  __device__ __forceinline__ uint32_t v(int dt) const { return v0 ^ static_cast<uint32_t>(dt << 5); }
};
__device__ __forceinline__ SparseLane sparse_lane(int hl, int gq) {
  SparseLane o;
  o.k0 = hl * kRowBytes + ((gq ^ swz(hl)) << 4);
  const int vr = 4 * gq + (hl >> 2);
  o.v0 = vr * kRowBytes + ((((hl & 3) >> 1) ^ swz(vr)) << 4) + ((hl & 1) << 3);
  return o;
}

// LDS bytes of a window's union list beside the ring: the member mask and the
// list entry of every key block (8 bytes per block) and the list length,
// rounded to 16 bytes
__host__ __device__ constexpr size_t sparse_list_bytes(int nb) {
  return 8 * static_cast<size_t>(nb) + 16;
}

// ---------------------------------------------------------------------------
// The union of the blocks a window's tokens attend (sparse kernels)
// ---------------------------------------------------------------------------
// Blocks attended by the query at position i: the initial blocks
// 0 .. n_init-1, the causal block window qb-n_local+1 .. qb (qb = i / 64)
// and its selected entries (news summary, Technical Mechanism; skill page,
// Step 2, sliding_attention made causal).  Entries outside [0, qb] are
// ignored and duplicates count once.  The list holds, ascending by block,
// entry = block | (16-bit member mask of the window's tokens) << 16.  bmask
// and blist are LDS arrays of at least qb_last + 1 entries.  All threads of
// the workgroup call this; it ends with a barrier and returns the length.
template <int NT>
__device__ __forceinline__ int build_union_list(uint32_t* bmask, int* blist, int* n_list, const int32_t* blk_idx,
                                                size_t bg, int r0, int off, int qb_last, const AttnShape& s, int wave,
                                                int lane) {
  for (int j = threadIdx.x; j <= qb_last; j += NT) bmask[j] = 0u;
  __syncthreads();
  const int per = s.topk + s.n_init + s.n_local;
  for (int e = threadIdx.x; e < kWin * per; e += NT) {
    const int tok = e / per, slot = e - tok * per;
    const int r = r0 + tok;
    if (r >= s.S_q) continue;
    const int i = off + r, qb = i / kBS;
    int j;
    if (slot < s.topk) {
      j = blk_idx[(bg * s.S_q + r) * s.topk + slot];
    } else {
      const int f = slot - s.topk;
      j = f < s.n_init ? f : qb - (f - s.n_init);
    }
    if (j >= 0 && j <= qb) atomicOr(&bmask[j], 1u << tok);
  }
  __syncthreads();
  if (wave == 0) {
    int cnt = 0;
    for (int base = 0; base <= qb_last; base += 64) {
      const int j = base + lane;
      const uint32_t mk = j <= qb_last ? bmask[j] : 0u;
      const uint64_t bal = __ballot(mk != 0u);
      if (mk) blist[cnt + mask_rank(bal)] = static_cast<int>(static_cast<uint32_t>(j) | (mk << 16));
      cnt += __popcll(bal);
    }
    if (lane == 0) *n_list = cnt;
  }
  __syncthreads();
  return *n_list;
}

// Stream list entries [e_lo, e_hi) through the 4-stage ring in pairs: the
// ring holds the pair being multiplied (2 stages) and the next pair in flight
// (the other 2); one barrier per pair.  on_pair(stg, js, cur0, cur1) gets the
// two stages, their blocks and their list entries (cur1 = 0 past the end).
// Waves 0 .. ISSUERS-1 issue the direct-to-LDS loads (64 KB per pair): with
// 16 waves each issuing 4, the CU moved 64 KB in about 3200 clocks in a
// probe, with 4 waves each issuing 8 in about half that per byte; the sparse
// forward uses 8 issuers (about 2% faster than 16 at 32k and 8k, 2 issuers 8%
// slower), the others start on their items at once.
// FRESH_DMA rebuilds the lane's DMA offsets at every issue from a lane id the
// compiler cannot hoist.  A kernel at its register limit would otherwise
// spill them and reload each from scratch just before its loads; the vmcnt
// wait for that reload also waits for the loads issued before it, which
// serialises the issue.
template <int WAVES, bool FRESH_DMA = false, int ISSUERS = WAVES, typename Src, typename Entry, typename F>
__device__ __forceinline__ void stream_pairs(unsigned char* smem, const Src& src, int e_lo, int e_hi,
                                             Entry entry_at, int wave, int lane, F&& on_pair) {
  static_assert(kStages == 4, "two pairs of stages");
  // the wave index in a scalar register: the stage addresses the loads write
  // to (M0) are then scalar arithmetic, not a vector value read back per load
  wave = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ring = lds_addr(smem);
  const bool issuer = wave < ISSUERS;
  const DmaLane<ISSUERS> dl_kept = dma_lane<ISSUERS>(wave % ISSUERS, lane);
  auto dl_fresh = [&]() { return FRESH_DMA ? dma_lane<ISSUERS>(wave % ISSUERS, lane_id_opaque()) : dl_kept; };
  const int nseg = e_hi - e_lo;
  auto seg_at = [&](int x) -> uint32_t { return x < nseg ? entry_at(e_lo + x) : 0u; };
  const int npair = (nseg + 1) / 2;
  uint32_t cur0 = __builtin_amdgcn_readfirstlane(seg_at(0)), cur1 = __builtin_amdgcn_readfirstlane(seg_at(1));
  uint32_t nxt0 = __builtin_amdgcn_readfirstlane(seg_at(2)), nxt1 = __builtin_amdgcn_readfirstlane(seg_at(3));
  if (issuer && nseg > 0) stage_src<ISSUERS>(ring, src, cur0 & 0xffffu, dl_fresh(), wave % ISSUERS, lane);
  if (issuer && nseg > 1) stage_src<ISSUERS>(ring + kStageBytes, src, cur1 & 0xffffu, dl_fresh(), wave % ISSUERS, lane);
  for (int pi = 0; pi < npair; ++pi) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // pair pi is in LDS; every wave is done with pair pi - 1
    const int half = (pi & 1) * 2;  // first stage of pair pi
    if (issuer && 2 * pi + 2 < nseg) {
      stage_src<ISSUERS>(ring + (half ^ 2) * kStageBytes, src, nxt0 & 0xffffu, dl_fresh(), wave % ISSUERS, lane);
      if (2 * pi + 3 < nseg)
        stage_src<ISSUERS>(ring + ((half ^ 2) + 1) * kStageBytes, src, nxt1 & 0xffffu, dl_fresh(), wave % ISSUERS, lane);
    }
    const unsigned char* stg[2] = {smem + half * kStageBytes, smem + (half + 1) * kStageBytes};
    const int js[2] = {static_cast<int>(cur0 & 0xffffu), static_cast<int>(cur1 & 0xffffu)};
    on_pair(stg, js, cur0, cur1);
    cur0 = nxt0;
    cur1 = nxt1;
    nxt0 = __builtin_amdgcn_readfirstlane(seg_at(2 * pi + 4));
    nxt1 = __builtin_amdgcn_readfirstlane(seg_at(2 * pi + 5));
  }
}

// ---------------------------------------------------------------------------
// The sparse item: one token (16 heads in the MFMA columns) over one or two
// attended 64-key blocks staged in the ring (forward, compressed branch and
// the fused decode kernel).  Online softmax in log2 units.
// ---------------------------------------------------------------------------
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

// Half-block pipeline: the same online softmax taken over 32-key halves of
// the attended blocks (half i = keys 32*(i%2) .. 32*(i%2)+31 of block i/2:
// S^T tiles 2*(i%2) and 2*(i%2)+1, and exactly k-step i%2 of O^T += V^T P^T).
// Each half's exp work is issued between the MFMAs of the next half's
// scores, and the next half's max between the MFMAs of this half's P V, so
// one wave keeps its matrix core busy during its own softmax.  The rescale
// decision stays per half (exact: a half's P is formed only after every
// earlier half has been accumulated at the running max it was scaled by).
__device__ __forceinline__ void qk_half(floatx4 (&sc)[2], const SparseState& st, const SparseLane& ln,
                                        const unsigned char* kbuf, int h) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 k0 = as_bf16x8(load16(kbuf + ln.k(ks) + (2 * h) * 16 * kRowBytes));
    const bf16x8 k1 = as_bf16x8(load16(kbuf + ln.k(ks) + (2 * h + 1) * 16 * kRowBytes));
    sc[0] = mfma_16x16x32(k0, st.qf[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : sc[0]);
    sc[1] = mfma_16x16x32(k1, st.qf[ks], ks == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : sc[1]);
  }
}

// keys past the token (only in the block holding its position) get -inf;
// lane (hl, gq) holds keys 16*kt + 4*gq + e2 of the block, kt = 2h + t
__device__ __forceinline__ void mask_half(floatx4 (&sc)[2], int first, int h) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      if (16 * (2 * h + t) + e2 > first) sc[t][e2] = -INFINITY;
}

// Maxima for the online softmax: IEEE maximum (v_maximum3_f32), which needs
// no quieting of MFMA results first (fmaxf adds a v_max of each input with
// itself); NaN scores (only from NaN inputs) propagate.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float max_half(const floatx4 (&sc)[2]) {
  return vmax(vmax(vmax(sc[0][0], sc[0][1]), vmax(sc[0][2], sc[0][3])),
              vmax(vmax(sc[1][0], sc[1][1]), vmax(sc[1][2], sc[1][3])));
}

// maximum over lanes l, l^16 and l^32 (the 4 lanes holding a head's keys)
__device__ __forceinline__ float vmax_lanes(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return vmax(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// running max update when the half's max (log2 units) passes it by the slack
__device__ __forceinline__ void rescale_half(SparseState& st, float mx) {
  const bool grow = mx > st.m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mn = grow ? mx : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);  // m = -inf on a row's first half: 0
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
    st.m = mn;
  }
}

// P of a half as the B operand of its P V k-step (slots 0..3: tile 2h,
// slots 4..7: tile 2h+1), and its row sum
__device__ __forceinline__ bf16x8 softmax_half(SparseState& st, const floatx4 (&sc)[2], float sl2) {
  const float nm = -st.m;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[e >> 2][e & 3], sl2, nm));
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  return as_bf16x8(u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                         pack_bf16x2(p[6], p[7])});
}

// O^T += V^T P^T for k-step h (keys 32h .. 32h+31): the V^T operand of lane
// (hl, gq) is keys 32h + 4*gq + {0..3} and 32h + 16 + 4*gq + {0..3} of dim 16*dt + hl
template <int VF = 2>
__device__ __forceinline__ void pv_half(SparseState& st, const SparseLane& ln, const unsigned char* vbuf, bf16x8 pf,
                                        int h) {
#pragma unroll
  for (int d0 = 0; d0 < 8; d0 += VF) {
    bf16x8 vf[VF];
#pragma unroll
    for (int dd = 0; dd < VF; ++dd) {
      const unsigned char* p = vbuf + ln.v(d0 + dd) + h * 32 * kRowBytes;
      vf[dd] = __builtin_shufflevector(lds_read_tr(p), lds_read_tr(p + 16 * kRowBytes), 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int dd = 0; dd < VF; ++dd) st.o[d0 + dd] = mfma_16x16x32(vf[dd], pf, st.o[d0 + dd]);
  }
}

// One pipeline step: the next half's scores (nxt, keys 32*hn.. of stage kn)
// under the exp work of the current half (cur), then the current half's P V
// (stage kc, k-step hc) under the next half's max.  MASK: the next half's
// block may hold keys past the token (mask_n, wave-uniform; first_n: see
// mask_half).
template <bool MASK>
__device__ __forceinline__ void half_step(SparseState& st, const SparseLane& ln, const floatx4 (&cur)[2],
                                          floatx4 (&nxt)[2], const unsigned char* kc, int hc,
                                          const unsigned char* kn, int hn, bool mask_n, int first_n, float sl2) {
  qk_half(nxt, st, ln, kn, hn);
  const bf16x8 pf = softmax_half(st, cur, sl2);
  pv_half(st, ln, kc + kTileBytes, pf, hc);
  if constexpr (MASK) {
    if (mask_n) mask_half(nxt, first_n, hn);
  }
  rescale_half(st, vmax_lanes(max_half(nxt)) * sl2);
}

// The wave's token over one or two attended blocks (stages ka, then kb if
// two), as one half-block pipeline.  MASK: a block may hold keys past the
// token (only its own block does): ma / mb (wave-uniform) say which, fa / fb
// are their mask offsets.
template <bool MASK>
__device__ __forceinline__ void sparse_blocks(SparseState& st, const SparseLane& ln, const unsigned char* ka,
                                              const unsigned char* kb, bool two, bool ma, bool mb, int fa, int fb,
                                              float sl2) {
  floatx4 a[2], b[2];
  qk_half(a, st, ln, ka, 0);
  if constexpr (MASK) {
    if (ma) mask_half(a, fa, 0);
  }
  rescale_half(st, vmax_lanes(max_half(a)) * sl2);
  half_step<MASK>(st, ln, a, b, ka, 0, ka, 1, ma, fa, sl2);
  const unsigned char* kl = ka;  // block of the last half
  if (two) {
    half_step<MASK>(st, ln, b, a, ka, 1, kb, 0, mb, fb, sl2);
    half_step<MASK>(st, ln, a, b, kb, 0, kb, 1, mb, fb, sl2);
    kl = kb;
  }
  pv_half(st, ln, kl + kTileBytes, softmax_half(st, b, sl2), 1);
}

// The wave's token over one streamed pair of stages (blocks js[0], js[1]):
// m0 / m1 say whether it attends each (wave-uniform).  A block that holds
// keys past the token (its own block) takes the masked pipeline.
__device__ __forceinline__ void attend_pair(SparseState& st, const SparseLane& spl, const unsigned char* const* stg,
                                            const int* js, bool m0, bool m1, int lane, float sl2) {
  const int lim = __builtin_amdgcn_readfirstlane(st.lim);
  const bool d0 = js[0] * kBS + kBS - 1 > lim, d1 = js[1] * kBS + kBS - 1 > lim;
  const int f0 = st.lim - js[0] * kBS - 4 * (lane >> 4), f1 = st.lim - js[1] * kBS - 4 * (lane >> 4);
  if (m0 || m1) {
    const unsigned char* ka = m0 ? stg[0] : stg[1];
    if ((m0 && d0) || (m1 && d1))
      sparse_blocks<true>(st, spl, ka, stg[1], m0 && m1, m0 ? d0 : d1, d1, m0 ? f0 : f1, f1, sl2);
    else
      sparse_blocks<false>(st, spl, ka, stg[1], m0 && m1, false, false, 0, 0, sl2);
  }
}


}  // namespace infv2
