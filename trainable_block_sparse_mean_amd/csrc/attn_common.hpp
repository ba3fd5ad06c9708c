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

}  // namespace infv2
