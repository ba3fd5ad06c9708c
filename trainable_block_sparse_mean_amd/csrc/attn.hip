// Block-sparse and dense attention forward for gfx950.
//
// Sparse: news summary "Technical Mechanism" (attention only on the selected
// key-value blocks) plus the initial blocks and a causal block-granular
// sliding window (skill page "Infllm V2 Dense Sparse Switchable Attention",
// Step 2 sliding_attention, made causal per Practical Guidance, When NOT to
// Use).  Dense: skill page, Step 1 (softmax of scaled products, weighted sum
// of values).
//
// Work unit: one workgroup = one KV group of one batch entry x a window of
// W consecutive query tokens; 4 waves, each owning T tokens.  For every
// token, the 16 query heads of the group are the N = 16 columns of a
// 16x16x32 bf16 MFMA, so no GQA head ever re-reads K/V on its own.
//   * The workgroup builds the union of the blocks its tokens attend (a
//     per-block bitmask of member tokens in LDS, compacted to an ascending
//     list), and streams each block of the union once through LDS.
//   * Each wave reads a block's K / V fragments from LDS once and applies
//     them to each of its tokens that attends the block (S^T = K Q^T, then
//     O^T += V^T P^T), so the LDS read of a fragment is shared by the member
//     tokens of the wave.
//   * S^T (keys x heads) leaves every lane with one head and four keys, so
//     the online softmax needs only two cross-lane steps per row, and its
//     output is already the B operand of V^T P^T once the 32 keys of a
//     k-step are taken in the order the lanes hold them.  The matching V^T
//     operand is read straight from V's natural [key][dim] rows with the
//     gfx950 transposing LDS read (ds_read_b64_tr_b16: each 16-lane group
//     turns a 4-key x 16-dim tile into one 4-key column per lane).
//   * K and V blocks go global -> LDS with asynchronous direct-to-LDS loads
//     (global_load_lds_dwordx4) into a double buffer, so the next block is in
//     flight while the current one is multiplied.  LDS rows are 256 bytes with
//     their 16-byte chunks XOR-swizzled by row, which keeps both the 16-row
//     K reads and the 8-row transposing V reads free of bank conflicts.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kWaves = 4;
constexpr int kRowBytes = kD * 2;                 // one K or V row in LDS
constexpr int kTileBytes = kBS * kRowBytes;       // one 64-key block of K (or V)
constexpr int kStageBytes = 2 * kTileBytes;       // K + V of one block
constexpr int kStages = 2;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16-byte chunk slot of chunk c in LDS row r: c ^ swz(r).  Any 16 consecutive
// rows get 16 distinct slots (conflict-free 16-lane K reads); any 8 rows of an
// aligned group of 8 get distinct 32-byte pairs (conflict-free V reads).
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Issue the direct-to-LDS loads of key block j (rows clamped to S_k - 1; the
// clamped keys are masked, and they hold finite data) into one stage buffer.
// Each wave moves 4 K and 4 V chunks of 4 rows (1 KB = 64 lanes x 16 B).
__device__ __forceinline__ void stage_block(unsigned char* stage, const uint16_t* kg, const uint16_t* vg,
                                            int j, int S_k, int wave, int lane) {
  const int sub = lane >> 4;    // row within the 4-row chunk
  const int slot = lane & 15;   // LDS chunk slot this lane fills
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int cc = wave * 4 + n;            // 4-row chunk 0..15
    const int row = cc * 4 + sub;
    const int grow = min(j * kBS + row, S_k - 1);
    const size_t off = static_cast<size_t>(grow) * kD + (slot ^ swz(row)) * 8;
    __builtin_amdgcn_global_load_lds((global_void*)(kg + off), (lds_void*)(stage + cc * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void*)(vg + off), (lds_void*)(stage + kTileBytes + cc * 1024), 16, 0, 0);
  }
}

template <int T, bool DENSE>
__global__ __launch_bounds__(256, 1) void attn_window_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             const int32_t* __restrict__ blk_idx,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse, AttnShape s) {
  constexpr int W = kWaves * T;
  extern __shared__ __align__(1024) unsigned char smem[];
  uint32_t* bmask = reinterpret_cast<uint32_t*>(smem + kStages * kStageBytes);  // [NB], sparse only
  int* blist = reinterpret_cast<int*>(bmask + s.NB);                           // [NB], sparse only
  __shared__ int n_list;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15;
  const int gq = lane >> 4;
  const int nwin = (s.S_q + W - 1) / W;
  const int win = nwin - 1 - static_cast<int>(blockIdx.x);  // latest (heaviest) windows first
  const int g = blockIdx.y % s.H_kv;
  const int b = blockIdx.y / s.H_kv;
  const size_t bg = static_cast<size_t>(b) * s.H_kv + g;
  const int r0 = win * W;
  const int off = s.S_k - s.S_q;
  const int i_last = off + min(r0 + W, s.S_q) - 1;
  const int qb_last = i_last / kBS;
  const uint16_t* kg = k + bg * s.S_k * kD;
  const uint16_t* vg = v + bg * s.S_k * kD;

  // ---- the union of attended blocks ---------------------------------------
  int nblk;
  if constexpr (DENSE) {
    nblk = s.causal ? qb_last + 1 : s.NB;
  } else {
    for (int j = threadIdx.x; j <= qb_last; j += 256) bmask[j] = 0u;
    __syncthreads();
    const int per = s.topk + s.n_init + s.n_local;
    for (int e = threadIdx.x; e < W * per; e += 256) {
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
        if (mk) blist[cnt + mask_rank(bal)] = j;
        cnt += __popcll(bal);
      }
      if (lane == 0) n_list = cnt;
    }
    __syncthreads();
    nblk = n_list;
  }

  // first block in flight while the queries load
  if (nblk > 0) stage_block(smem, kg, vg, DENSE ? 0 : blist[0], s.S_k, wave, lane);

  // ---- per-token state (this wave's T tokens) -------------------------------
  bf16x8 qf[T][4];
  floatx4 o[T][8];
  float m[T], l[T], lr[T];  // l: this lane's fp32 row sum, lr: of the bf16-rounded P
  int ipos[T];
  uint32_t valid_mask = 0;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int r = r0 + wave * T + t;
    const bool valid = r < s.S_q;
    valid_mask |= valid ? (1u << t) : 0u;
    ipos[t] = off + r;
    const int h = g * s.G + hl;
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + h) * s.S_q + r) * kD + gq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[t][ks] = (valid && hl < s.G) ? as_bf16x8(load16(qrow + ks * 32)) : bf16x8{};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    m[t] = -INFINITY;
    l[t] = 0.f;
    lr[t] = 0.f;
  }

  // ---- stream the blocks -----------------------------------------------------
  for (int e = 0; e < nblk; ++e) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block e is in LDS; every wave is done with block e - 1
    if (e + 1 < nblk)
      stage_block(smem + ((e + 1) & 1) * kStageBytes, kg, vg, DENSE ? e + 1 : blist[e + 1], s.S_k, wave, lane);

    const int j = DENSE ? e : blist[e];
    uint32_t wm;
    if constexpr (DENSE) {
      wm = 0u;
#pragma unroll
      for (int t = 0; t < T; ++t)
        if ((valid_mask >> t & 1u) && (!s.causal || j * kBS <= ipos[t])) wm |= 1u << t;
    } else {
      wm = (bmask[j] >> (wave * T)) & ((1u << T) - 1u);
    }
    if (wm == 0u) continue;
    const unsigned char* kbuf = smem + (e & 1) * kStageBytes;
    const unsigned char* vbuf = kbuf + kTileBytes;

    // S^T[key][head] = K Q^T for every member token
    floatx4 sacc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sacc[t][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int row = 16 * kt + hl;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = as_bf16x8(load16(kbuf + row * kRowBytes + (((ks * 4 + gq) ^ swz(row)) << 4)));
#pragma unroll
        for (int t = 0; t < T; ++t)
          if (wm >> t & 1u) sacc[t][kt] = mfma_16x16x32(a, qf[t][ks], sacc[t][kt]);
      }
    }

    // online softmax (log2 domain).  P is rounded to bf16 for the PV product.
    // Row sums stay per lane (each lane holds 16 of a head's 64 keys) and are
    // reduced across the four lanes of a head once, after the last block: l
    // sums the fp32 P (for the log-sum-exp), lr the rounded P (O is divided
    // by lr, so its weights are exactly those the MFMA applied).
    bf16x8 pf[T][2];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (!(wm >> t & 1u)) continue;
      const int lim = DENSE && !s.causal ? s.S_k - 1 : min(ipos[t], s.S_k - 1);
      const bool need_mask = j * kBS + kBS - 1 > lim;
      float z[16];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float zz = sacc[t][kt][e2] * s.scale_log2;
          if (need_mask && j * kBS + 16 * kt + 4 * gq + e2 > lim) zz = -INFINITY;
          z[kt * 4 + e2] = zz;
          mx = fmaxf(mx, zz);
        }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mn = fmaxf(m[t], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[t] - mn);  // m = -inf on the first block: 0
      uint32_t pw[8];
      float rs = 0.f, rsr = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < 8; ++c2) {
        const float p0 = __builtin_amdgcn_exp2f(z[2 * c2] - mn);
        const float p1 = __builtin_amdgcn_exp2f(z[2 * c2 + 1] - mn);
        pw[c2] = pack_bf16x2(p0, p1);
        rs += p0 + p1;
        rsr += bf16_lo(pw[c2]) + bf16_hi(pw[c2]);
      }
      l[t] = l[t] * alpha + rs;
      lr[t] = lr[t] * alpha + rsr;
      m[t] = mn;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
      // k-step s2 takes S^T tiles 2*s2 (slots 0..3) and 2*s2+1 (slots 4..7)
      pf[t][0] = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
      pf[t][1] = as_bf16x8(u32x4{pw[4], pw[5], pw[6], pw[7]});
    }

    // O^T[dim][head] += V^T P^T; the V^T operand of lane (hl, gq) for k-step
    // s2 is keys 32*s2 + 4*gq + {0..3} and 32*s2 + 16 + 4*gq + {0..3} of dim
    // 16*dt + hl: two transposing reads of 4-key x 16-dim tiles
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x4 half[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = 32 * s2 + 16 * hh + 4 * gq + (hl >> 2);
          const int chunk = 2 * dt + ((hl & 3) >> 1);
          half[hh] = lds_read_tr(vbuf + row * kRowBytes + ((chunk ^ swz(row)) << 4) + ((hl & 1) << 3));
        }
        const bf16x8 a = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int t = 0; t < T; ++t)
          if (wm >> t & 1u) o[t][dt] = mfma_16x16x32(a, pf[t][s2], o[t][dt]);
      }
    }
  }

  // ---- epilogue ---------------------------------------------------------------
#pragma unroll
  for (int t = 0; t < T; ++t) {
    l[t] += shfl_xor(l[t], 16);
    l[t] += shfl_xor(l[t], 32);
    lr[t] += shfl_xor(lr[t], 16);
    lr[t] += shfl_xor(lr[t], 32);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (!(valid_mask >> t & 1u) || hl >= s.G) continue;
    const int r = r0 + wave * T + t;
    const int h = g * s.G + hl;
    const float inv = 1.f / lr[t];
    uint16_t* orow = out + (static_cast<size_t>(b * s.H_q + h) * s.S_q + r) * kD + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x2 w = {pack_bf16x2(o[t][dt][0] * inv, o[t][dt][1] * inv),
                       pack_bf16x2(o[t][dt][2] * inv, o[t][dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * dt) = w;
    }
    if (lse && gq == 0) lse[static_cast<size_t>(b * s.H_q + h) * s.S_q + r] = (m[t] + log2f(l[t])) * kLn2;
  }
}

constexpr int kTokPerWave = 4;

size_t attn_workspace_bytes(const AttnShape&) { return 0; }

template <bool DENSE>
static hipError_t launch_window(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* blk_idx,
                                uint16_t* out, float* lse, const AttnShape& s, hipStream_t stream) {
  constexpr int W = kWaves * kTokPerWave;
  const dim3 grid((s.S_q + W - 1) / W, s.B * s.H_kv);
  const size_t lds = kStages * kStageBytes + (DENSE ? 0 : 2 * sizeof(int) * static_cast<size_t>(s.NB));
  hipLaunchKernelGGL((attn_window_kernel<kTokPerWave, DENSE>), grid, dim3(256), lds, stream, q, k, v, blk_idx,
                     out, lse, s);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* blk_idx, uint16_t* out, float* lse,
                              const AttnShape& s, void*, hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  return launch_window<false>(q, k, v, blk_idx, out, lse, s, stream);
}

hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, const AttnShape& s, void*, hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  return launch_window<true>(q, k, v, nullptr, out, lse, s, stream);
}

}  // namespace infv2
