// Key compression: per-block means of K (skill page "Infllm V2 Dense Sparse
// Switchable Attention", Step 2, compressed_attention — zero padding to a
// multiple of the block size, mean over each block's tokens).
//
// HBM-bound: every key byte is read once and 1/64 of it is written.  One
// wave per compressed block; lane l owns dims 2l and 2l+1, so each row of the
// block is one coalesced 256-byte wave load.  Sums are accumulated in fp64,
// which is exact for bf16 inputs whose magnitudes span fewer than ~2^39, so
// the rounded mean does not depend on the summation order.
#include "common.hpp"
#include "kernels.hpp"

namespace infv2 {

__global__ __launch_bounds__(256) void compress_k_kernel(const uint16_t* __restrict__ k,
                                                         uint16_t* __restrict__ k_cmp,
                                                         int S_k, int NB) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + wave;
  if (j >= NB) return;
  const size_t head = blockIdx.y;  // b * H_kv + g
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(k + (head * S_k + static_cast<size_t>(j) * kBS) * kD) + lane;
  const int n = min(kBS, S_k - j * kBS);
  double s0 = 0.0, s1 = 0.0;
  if (n == kBS) {
#pragma unroll 16
    for (int t = 0; t < kBS; ++t) {
      const uint32_t w = __builtin_nontemporal_load(src + t * (kD / 2));
      s0 += static_cast<double>(bf16_lo(w));
      s1 += static_cast<double>(bf16_hi(w));
    }
  } else {
    for (int t = 0; t < n; ++t) {
      const uint32_t w = src[t * (kD / 2)];
      s0 += static_cast<double>(bf16_lo(w));
      s1 += static_cast<double>(bf16_hi(w));
    }
  }
  // the divisor is the block size also for the zero-padded tail block
  const uint32_t packed = f64_to_bf16_bits(s0 * (1.0 / kBS)) | (f64_to_bf16_bits(s1 * (1.0 / kBS)) << 16);
  reinterpret_cast<uint32_t*>(k_cmp + (head * NB + j) * kD)[lane] = packed;
}

// Paged cache: the compressed key of every block of sequence b that is
// complete at new length L = seq_keys(b) but was not at old_len[b] (blocks
// floor(old/64) .. floor(L/64) - 1), from the block's page.  One wave per
// (block slot, KV head); slot x of sequence b is block floor(old/64) + x.
// Partial blocks are left alone: the selection only scores complete blocks.
__global__ __launch_bounds__(256) void compress_append_kernel(const uint16_t* __restrict__ k_pages,
                                                              uint16_t* __restrict__ k_cmp, AttnShape s,
                                                              const int* __restrict__ old_len, int max_new) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int x = blockIdx.x * 4 + wave;
  const int b = blockIdx.y / s.H_kv, g = blockIdx.y % s.H_kv;
  if (x >= max_new) return;
  const int L = seq_keys(s, b);
  const int first = min(max(old_len[b], 0), L) / kBS;
  const int j = first + x;
  if (j >= L / kBS) return;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(k_pages + page_rows(s, b, g, j)) + lane;
  double s0 = 0.0, s1 = 0.0;
#pragma unroll 16
  for (int t = 0; t < kBS; ++t) {
    const uint32_t w = __builtin_nontemporal_load(src + t * (kD / 2));
    s0 += static_cast<double>(bf16_lo(w));
    s1 += static_cast<double>(bf16_hi(w));
  }
  const uint32_t packed = f64_to_bf16_bits(s0 * (1.0 / kBS)) | (f64_to_bf16_bits(s1 * (1.0 / kBS)) << 16);
  reinterpret_cast<uint32_t*>(k_cmp + ((static_cast<size_t>(b) * s.H_kv + g) * s.NB + j) * kD)[lane] = packed;
}

hipError_t launch_compress_append(const uint16_t* k_pages, const AttnShape& s, const int* old_len,
                                  uint16_t* k_cmp, int max_new, hipStream_t stream) {
  if (s.B == 0 || max_new <= 0) return hipSuccess;
  dim3 grid((max_new + 3) / 4, s.B * s.H_kv);
  hipLaunchKernelGGL(compress_append_kernel, grid, dim3(256), 0, stream, k_pages, k_cmp, s, old_len, max_new);
  return hipGetLastError();
}

hipError_t launch_compress_k(const uint16_t* k, uint16_t* k_cmp, int B, int H_kv, int S_k,
                             hipStream_t stream) {
  const int NB = (S_k + kBS - 1) / kBS;
  if (NB == 0 || B == 0) return hipSuccess;
  dim3 grid((NB + 3) / 4, B * H_kv);
  hipLaunchKernelGGL(compress_k_kernel, grid, dim3(256), 0, stream, k, k_cmp, S_k, NB);
  return hipGetLastError();
}

}  // namespace infv2
