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
//     k-step are taken in the order the lanes hold them.  V is relaid out
//     once per call into that block-transposed, key-permuted order so the
//     V^T fragment of a lane is one 16-byte LDS read.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kWaves = 4;
constexpr int kKPitch = kD * 2 + 16;   // bytes per K row in LDS (pad: conflict-free 16-row reads)
constexpr int kVPitch = kBS * 2 + 16;  // bytes per V^T row in LDS
constexpr int kKBytes = kBS * kKPitch;
constexpr int kVBytes = kD * kVPitch;

// Key held in position p (0..63) of a relaid V^T row: within each 32-key
// group, lane quad gq's eight slots are keys 4gq..4gq+3 and 16+4gq..16+4gq+3.
__host__ __device__ constexpr int vt_key_of_pos(int p) {
  return 32 * (p >> 5) + (((p & 7) < 4) ? (4 * ((p & 31) >> 3) + (p & 7))
                                        : (16 + 4 * ((p & 31) >> 3) + (p & 7) - 4));
}

// vt[bg][blk][d][p] = v[bg][blk*64 + vt_key_of_pos(p)][d] (0 beyond S_k)
__global__ __launch_bounds__(256) void v_relayout_kernel(const uint16_t* __restrict__ v,
                                                         uint16_t* __restrict__ vt, int S_k, int NB) {
  __shared__ __align__(16) uint16_t tile[kBS][kD + 8];
  const int blk = blockIdx.x;
  const size_t bg = blockIdx.y;
  const int nvalid = min(kBS, S_k - blk * kBS);
  for (int c = threadIdx.x; c < kBS * kD / 8; c += 256) {
    const int key = c >> 4, col = (c & 15) * 8;
    const u32x4 val = key < nvalid ? load16(v + (bg * S_k + static_cast<size_t>(blk) * kBS + key) * kD + col)
                                   : u32x4{0u, 0u, 0u, 0u};
    store16(&tile[key][col], val);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < kBS * kD / 8; c += 256) {
    const int d = c >> 3, pc = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k0 = vt_key_of_pos(pc * 8 + 2 * e), k1 = vt_key_of_pos(pc * 8 + 2 * e + 1);
      w[e] = static_cast<uint32_t>(tile[k0][d]) | (static_cast<uint32_t>(tile[k1][d]) << 16);
    }
    store16(vt + ((bg * NB + blk) * kD + d) * kBS + pc * 8, u32x4{w[0], w[1], w[2], w[3]});
  }
}

template <int T, bool DENSE>
__global__ __launch_bounds__(256, 1) void attn_window_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ vt,
                                                             const int32_t* __restrict__ blk_idx,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse, AttnShape s) {
  constexpr int W = kWaves * T;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kbuf = smem;
  unsigned char* vbuf = smem + kKBytes;
  uint32_t* bmask = reinterpret_cast<uint32_t*>(smem + kKBytes + kVBytes);  // [NB], sparse only
  int* blist = reinterpret_cast<int*>(bmask + s.NB);                        // [NB], sparse only
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

    __syncthreads();  // every wave is done with the previous block
    for (int c = threadIdx.x; c < kBS * kD / 8; c += 256) {
      const int row = c >> 4, col = c & 15;
      const int kpos = j * kBS + row;
      const u32x4 kv = kpos < s.S_k ? load16(k + (bg * s.S_k + kpos) * kD + col * 8) : u32x4{0u, 0u, 0u, 0u};
      store16(kbuf + row * kKPitch + col * 16, kv);
      const int d = c >> 3, pc = c & 7;
      store16(vbuf + d * kVPitch + pc * 16, load16(vt + ((bg * s.NB + j) * kD + d) * kBS + pc * 8));
    }
    __syncthreads();
    if (wm == 0u) continue;

    // S^T[key][head] = K Q^T for every member token
    floatx4 sacc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sacc[t][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = as_bf16x8(load16(kbuf + (16 * kt + hl) * kKPitch + ks * 64 + gq * 16));
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
      const float alpha = exp2f(m[t] - mn);  // m = -inf on the first block: 0
      uint32_t pw[8];
      float rs = 0.f, rsr = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < 8; ++c2) {
        const float p0 = exp2f(z[2 * c2] - mn), p1 = exp2f(z[2 * c2 + 1] - mn);
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

    // O^T[dim][head] += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 a = as_bf16x8(load16(vbuf + (16 * dt + hl) * kVPitch + s2 * 64 + gq * 16));
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

size_t attn_workspace_bytes(const AttnShape& s) {
  return static_cast<size_t>(s.B) * s.H_kv * s.NB * kBS * kD * sizeof(uint16_t);
}

static hipError_t launch_relayout(const uint16_t* v, uint16_t* vt, const AttnShape& s, hipStream_t stream) {
  hipLaunchKernelGGL(v_relayout_kernel, dim3(s.NB, s.B * s.H_kv), dim3(256), 0, stream, v, vt, s.S_k, s.NB);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* blk_idx, uint16_t* out, float* lse,
                              const AttnShape& s, void* workspace, hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  uint16_t* vt = static_cast<uint16_t*>(workspace);
  hipError_t err = launch_relayout(v, vt, s, stream);
  if (err != hipSuccess) return err;
  constexpr int W = kWaves * kTokPerWave;
  const dim3 grid((s.S_q + W - 1) / W, s.B * s.H_kv);
  const size_t lds = kKBytes + kVBytes + 2 * sizeof(int) * static_cast<size_t>(s.NB);
  hipLaunchKernelGGL((attn_window_kernel<kTokPerWave, false>), grid, dim3(256), lds, stream, q, k, vt,
                     blk_idx, out, lse, s);
  return hipGetLastError();
}

hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, const AttnShape& s, void* workspace,
                             hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  uint16_t* vt = static_cast<uint16_t*>(workspace);
  hipError_t err = launch_relayout(v, vt, s, stream);
  if (err != hipSuccess) return err;
  constexpr int W = kWaves * kTokPerWave;
  const dim3 grid((s.S_q + W - 1) / W, s.B * s.H_kv);
  const size_t lds = kKBytes + kVBytes;
  hipLaunchKernelGGL((attn_window_kernel<kTokPerWave, true>), grid, dim3(256), lds, stream, q, k, vt,
                     nullptr, out, lse, s);
  return hipGetLastError();
}

}  // namespace infv2
