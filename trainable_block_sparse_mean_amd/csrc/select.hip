// Block selection: group-summed block scores + top-k.
//
// Scores: skill page "Infllm V2 Dense Sparse Switchable Attention",
// Architecture Overview (Hardware Kernel: log-sum-exp-normalised scores
// summed over the heads of a group) and Step 2 (compressed_attention: softmax
// of the scaled query / compressed-key products).  Selection: Step 2,
// selected_attention (top-k per query position) at block granularity (news
// summary, Technical Mechanism).
//
// A wave handles kTok consecutive query tokens of one KV head.  For each
// token the 16 heads of the group are the N dimension of a 16x16x32 bf16
// MFMA and the compressed keys the M dimension, so a tile of 16 block scores
// is 4 MFMAs (K = 128).  Each compressed-key fragment is loaded once per wave
// and applied to all of its tokens.  Pass 1 computes each head's log-sum-exp
// over the fully visible blocks with an online max; pass 2 recomputes the
// scores, normalises them and sums the heads with DPP row rotations (the 16
// lanes of a row hold the 16 heads of one block).  Group scores stay in LDS,
// never in HBM.  The top-k is an exact radix select on the fp32 bit patterns
// (non-negative floats order like their bits), then ties are taken lowest
// index first and the kept indices compacted in ascending order by ballot.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kSelWaves = 4;
constexpr int kSelTok = 4;                          // tokens per wave
constexpr int kSelWin = kSelWaves * kSelTok;        // tokens per workgroup
constexpr int kMaxCandIt = 32;                      // NB <= 2048: at most 32 candidates per lane

// sum over the 16 lanes of a DPP row (every lane receives the sum)
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}

// online (max, sum of exp2) of the two lanes l and l ^ off
__device__ __forceinline__ void lse_merge(float& m, float& l, int off) {
  const float mo = shfl_xor(m, off), lo = shfl_xor(l, off);
  const float mn = fmaxf(m, mo);
  l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + (mo == -INFINITY ? 0.f : lo * exp2f(mo - mn));
  m = mn;
}

__global__ __launch_bounds__(kSelWaves * 64) void select_blocks_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ kc,
                                                                       int32_t* __restrict__ blk_idx,
                                                                       float* __restrict__ blk_score,
                                                                       AttnShape s) {
  extern __shared__ float sig_all[];  // [kSelWin][sig_stride]
  // per-token stride: NB rounded up to whole 16-block tiles, so the tile
  // stores below stay inside each token's own row
  const int sig_stride = (s.NB + 15) & ~15;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15;   // head within the group (MFMA column)
  const int gq = lane >> 4;   // k-slot group / row quad
  const int g = blockIdx.y % s.H_kv;
  const int b = blockIdx.y / s.H_kv;
  const int r0 = blockIdx.x * kSelWin + wave * kSelTok;  // first token of this wave
  const int off = s.S_k - s.S_q;

  int nv[kSelTok];
  int nv_max = 0;
#pragma unroll
  for (int t = 0; t < kSelTok; ++t) {
    const int r = r0 + t;
    nv[t] = r < s.S_q ? (off + r + 1) / kBS : 0;
    nv_max = max(nv_max, nv[t]);
  }

  // ---- group scores -> LDS ------------------------------------------------
  if (nv_max > 0) {
    bf16x8 qf[kSelTok][4];
#pragma unroll
    for (int t = 0; t < kSelTok; ++t) {
      const int r = r0 + t;
      const uint16_t* qrow =
          q + (static_cast<size_t>(b * s.H_q + g * s.G + hl) * s.S_q + r) * kD + gq * 8;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[t][ks] = (r < s.S_q && hl < s.G) ? as_bf16x8(load16(qrow + ks * 32)) : bf16x8{};
    }
    const uint16_t* kbase = kc + static_cast<size_t>(b * s.H_kv + g) * s.NB * kD + gq * 8;
    const int ntile = (nv_max + 15) / 16;

    // pass 1: per-head log-sum-exp (log2 domain), each lane over its rows
    float m[kSelTok], l[kSelTok];
#pragma unroll
    for (int t = 0; t < kSelTok; ++t) {
      m[t] = -INFINITY;
      l[t] = 0.f;
    }
    for (int jt = 0; jt < ntile; ++jt) {
      const int jrow = min(jt * 16 + hl, s.NB - 1);
      bf16x8 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = as_bf16x8(load16(kbase + static_cast<size_t>(jrow) * kD + ks * 32));
#pragma unroll
      for (int t = 0; t < kSelTok; ++t) {
        floatx4 acc = mfma_16x16x32(kf[0], qf[t][0], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) acc = mfma_16x16x32(kf[ks], qf[t][ks], acc);
        float zmax = -INFINITY;
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jt * 16 + gq * 4 + e;
          z[e] = j < nv[t] ? acc[e] * s.scale_log2 : -INFINITY;
          zmax = fmaxf(zmax, z[e]);
        }
        if (zmax > -INFINITY) {
          const float mn = fmaxf(m[t], zmax);
          float add = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) add += exp2f(z[e] - mn);
          l[t] = l[t] * exp2f(m[t] - mn) + add;
          m[t] = mn;
        }
      }
    }
    float lse2[kSelTok];
#pragma unroll
    for (int t = 0; t < kSelTok; ++t) {
      lse_merge(m[t], l[t], 16);
      lse_merge(m[t], l[t], 32);
      lse2[t] = m[t] + log2f(l[t]);
    }

    // pass 2: normalised scores, summed over the heads of the group
    for (int jt = 0; jt < ntile; ++jt) {
      const int jrow = min(jt * 16 + hl, s.NB - 1);
      bf16x8 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = as_bf16x8(load16(kbase + static_cast<size_t>(jrow) * kD + ks * 32));
#pragma unroll
      for (int t = 0; t < kSelTok; ++t) {
        if (jt * 16 >= nv[t]) continue;
        floatx4 acc = mfma_16x16x32(kf[0], qf[t][0], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) acc = mfma_16x16x32(kf[ks], qf[t][ks], acc);
        floatx4 p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jt * 16 + gq * 4 + e;
          p[e] = row_sum16((j < nv[t] && hl < s.G) ? exp2f(acc[e] * s.scale_log2 - lse2[t]) : 0.f);
        }
        // lane (hl = 0, gq) stores the 4 group scores of blocks 16*jt + 4*gq + e
        if (hl == 0) *reinterpret_cast<floatx4*>(sig_all + (wave * kSelTok + t) * sig_stride + jt * 16 + gq * 4) = p;
      }
    }
  }
  __syncthreads();  // (each wave reads only its own tokens' scores; kept for clarity)

  if (s.topk == 0) return;

  // ---- top-k over the candidates n_init .. qb - n_local, one token at a time -
  for (int t = 0; t < kSelTok; ++t) {
    const int r = r0 + t;
    if (r >= s.S_q) break;
    const float* sig = sig_all + (wave * kSelTok + t) * sig_stride;
    const int qb = (off + r) / kBS;
    const int lo = s.n_init;
    const int hi = qb - s.n_local;
    const int nC = hi >= lo ? hi - lo + 1 : 0;
    const int kk = min(s.topk, nC);
    int32_t* out = blk_idx + (static_cast<size_t>(b * s.H_kv + g) * s.S_q + r) * s.topk;
    float* out_s = blk_score ? blk_score + (static_cast<size_t>(b * s.H_kv + g) * s.S_q + r) * s.topk : nullptr;

    if (nC <= s.topk) {  // every candidate is kept
      for (int e = lane; e < s.topk; e += 64) {
        out[e] = e < nC ? lo + e : -1;
        if (out_s) out_s[e] = e < nC ? sig[lo + e] : 0.f;
      }
      continue;
    }

    const int nIt = (nC + 63) / 64;
    uint32_t x[kMaxCandIt];
#pragma unroll
    for (int it = 0; it < kMaxCandIt; ++it) {
      const int c = it * 64 + lane;
      x[it] = (it < nIt && c < nC) ? __float_as_uint(sig[lo + c]) : 0u;
    }
    // validity of slot `it` of this lane: it * 64 + lane < nC
    auto valid = [&](int it) { return it * 64 + lane < nC; };

    // largest tt with #{x >= tt} >= kk is the kk-th largest value (bits 30..0;
    // the sign bit is clear for non-negative scores)
    uint32_t tt = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = tt | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int it = 0; it < kMaxCandIt; ++it)
        if (it < nIt) cnt += __popcll(__ballot(valid(it) && x[it] >= cand));
      if (cnt >= kk) tt = cand;
    }
    int n_gt = 0;
#pragma unroll
    for (int it = 0; it < kMaxCandIt; ++it)
      if (it < nIt) n_gt += __popcll(__ballot(valid(it) && x[it] > tt));
    const int need_eq = kk - n_gt;  // ties at tt, lowest indices first

    int eq_before = 0, n_out = 0;
#pragma unroll
    for (int it = 0; it < kMaxCandIt; ++it) {
      if (it < nIt) {
        const bool v = valid(it);
        const bool gt = v && x[it] > tt;
        const bool eq = v && x[it] == tt;
        const uint64_t eqm = __ballot(eq);
        const bool sel = gt || (eq && eq_before + mask_rank(eqm) < need_eq);
        eq_before += __popcll(eqm);
        const uint64_t selm = __ballot(sel);
        if (sel) {
          const int pos = n_out + mask_rank(selm);
          out[pos] = lo + it * 64 + lane;
          if (out_s) out_s[pos] = __uint_as_float(x[it]);
        }
        n_out += __popcll(selm);
      }
    }
    for (int e = kk + lane; e < s.topk; e += 64) {
      out[e] = -1;
      if (out_s) out_s[e] = 0.f;
    }
  }
}

hipError_t launch_select_blocks(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx,
                                float* blk_score, const AttnShape& s, hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  dim3 grid((s.S_q + kSelWin - 1) / kSelWin, s.B * s.H_kv);
  const size_t lds = static_cast<size_t>(kSelWin) * ((s.NB + 15) & ~15) * sizeof(float);
  hipLaunchKernelGGL(select_blocks_kernel, grid, dim3(64 * kSelWaves), lds, stream, q, k_cmp, blk_idx,
                     blk_score, s);
  return hipGetLastError();
}

}  // namespace infv2
