// Block selection: group-summed block scores + top-k.
//
// Scores: skill page "Infllm V2 Dense Sparse Switchable Attention",
// Architecture Overview (Hardware Kernel: log-sum-exp–normalised scores
// summed over the heads of a group) and Step 2 (compressed_attention: softmax
// of the scaled query / compressed-key products).  Selection: Step 2,
// selected_attention (top-k per query position) at block granularity (news
// summary, Technical Mechanism).
//
// One wave per (query token, KV group).  The 16 heads of the group are the
// N dimension of a 16x16x32 bf16 MFMA; the compressed keys are the M
// dimension, so a 16-block tile of scores is 4 MFMAs (K = 128 = 4 x 32).
// Pass 1 computes each head's log-sum-exp over the fully visible blocks with
// an online max; pass 2 recomputes the scores, normalises them and sums the
// heads with a butterfly over the 16 lanes that hold one block's heads.  The
// group scores stay in LDS (never in HBM); the top-k is an exact radix
// select on the fp32 bit patterns (non-negative floats order like their
// bits) followed by a lowest-index-first pass over the ties and an
// ascending compaction with ballots.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

constexpr int kSelWaves = 4;
constexpr int kMaxCandIt = 32;  // NB <= 2048: at most 32 candidates per lane

__global__ __launch_bounds__(256) void select_blocks_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ kc,
                                                            int32_t* __restrict__ blk_idx,
                                                            float* __restrict__ blk_score,
                                                            AttnShape s) {
  extern __shared__ float sig_all[];  // [kSelWaves][NB]
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15;   // head within the group (MFMA column)
  const int gq = lane >> 4;   // k-slot group / row quad
  const int g = blockIdx.y % s.H_kv;
  const int b = blockIdx.y / s.H_kv;
  const int r = blockIdx.x * kSelWaves + wave;
  const bool active = r < s.S_q;
  float* sig = sig_all + wave * s.NB;

  const int i = s.S_k - s.S_q + r;  // absolute position of the query
  const int nv = active ? (i + 1) / kBS : 0;
  const int qb = i / kBS;

  // ---- group scores -> LDS ------------------------------------------------
  if (active && nv > 0) {
    const int h = g * s.G + hl;
    bf16x8 qf[4];
    const uint16_t* qrow = q + (static_cast<size_t>(b * s.H_q + h) * s.S_q + r) * kD + gq * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = hl < s.G ? as_bf16x8(load16(qrow + ks * 32)) : bf16x8{};
    const uint16_t* kbase = kc + static_cast<size_t>(b * s.H_kv + g) * s.NB * kD + gq * 8;
    const int ntile = (nv + 15) / 16;

    // pass 1: per-head log-sum-exp (log2 domain), each lane over its rows
    float m = -INFINITY, l = 0.f;
    for (int jt = 0; jt < ntile; ++jt) {
      const int jrow = min(jt * 16 + hl, s.NB - 1);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma_16x16x32(as_bf16x8(load16(kbase + static_cast<size_t>(jrow) * kD + ks * 32)), qf[ks], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jt * 16 + gq * 4 + e;
        if (j < nv) {
          const float z = acc[e] * s.scale_log2;
          if (z > m) {
            l = l * exp2f(m - z) + 1.f;
            m = z;
          } else {
            l += exp2f(z - m);
          }
        }
      }
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float mo = shfl_xor(m, off);
      const float lo = shfl_xor(l, off);
      const float mn = fmaxf(m, mo);
      l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + (mo == -INFINITY ? 0.f : lo * exp2f(mo - mn));
      m = mn;
    }
    const float lse2 = m + log2f(l);

    // pass 2: normalised scores, summed over the heads of the group
    for (int jt = 0; jt < ntile; ++jt) {
      const int jrow = min(jt * 16 + hl, s.NB - 1);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma_16x16x32(as_bf16x8(load16(kbase + static_cast<size_t>(jrow) * kD + ks * 32)), qf[ks], acc);
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jt * 16 + gq * 4 + e;
        p[e] = (j < nv && hl < s.G) ? exp2f(acc[e] * s.scale_log2 - lse2) : 0.f;
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] += shfl_xor(p[e], off);
      }
      if (hl == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jt * 16 + gq * 4 + e;
          if (j < nv) sig[j] = p[e];
        }
      }
    }
  }
  __syncthreads();

  if (!active || s.topk == 0) return;  // no barriers below

  // ---- top-k over the candidates n_init .. qb - n_local ---------------------
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
    return;
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

  // largest t with #{x >= t} >= kk is the kk-th largest value (bits 30..0;
  // the sign bit is clear for non-negative scores)
  uint32_t t = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int it = 0; it < kMaxCandIt; ++it)
      if (it < nIt) cnt += __popcll(__ballot(valid(it) && x[it] >= cand));
    if (cnt >= kk) t = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int it = 0; it < kMaxCandIt; ++it)
    if (it < nIt) n_gt += __popcll(__ballot(valid(it) && x[it] > t));
  const int need_eq = kk - n_gt;  // ties at t, lowest indices first

  int eq_before = 0, n_out = 0;
#pragma unroll
  for (int it = 0; it < kMaxCandIt; ++it) {
    if (it < nIt) {
      const bool v = valid(it);
      const bool gt = v && x[it] > t;
      const bool eq = v && x[it] == t;
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

hipError_t launch_select_blocks(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx,
                                float* blk_score, const AttnShape& s, hipStream_t stream) {
  if (s.B == 0 || s.S_q == 0) return hipSuccess;
  dim3 grid((s.S_q + kSelWaves - 1) / kSelWaves, s.B * s.H_kv);
  const size_t lds = static_cast<size_t>(kSelWaves) * s.NB * sizeof(float);
  hipLaunchKernelGGL(select_blocks_kernel, grid, dim3(64 * kSelWaves), lds, stream, q, k_cmp,
                     blk_idx, blk_score, s);
  return hipGetLastError();
}

}  // namespace infv2
