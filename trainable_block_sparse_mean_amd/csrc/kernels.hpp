// Internal launch functions of the gfx950 kernels (called by api.hip after
// argument validation).  Shapes here are already checked: D = 128,
// block size 64, 1 <= G <= 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace infv2 {

struct AttnShape {
  int B, H_q, H_kv, S_q, S_k, G, NB;
  int topk, n_init, n_local;
  float scale_log2;  // softmax scale * log2(e)
  int causal;
  int nsplit;        // sparse: workgroups sharing one window's block list (1 = no split)
};

// Split-KV partials of the sparse kernel, in the workspace: for split s and
// query row (b, h, r), 128 unnormalised fp32 output values relative to the
// split's running max, then that max (log2 units) and the row sum (two
// padding floats keep rows 16-byte aligned).
constexpr int kPartFloats = 132;  // 128 + m + l, padded to 16 bytes

// number of splits the sparse kernel uses for a shape (1 for long queries)
int sparse_splits(int B, int H_kv, int S_q, int topk);

hipError_t launch_compress_k(const uint16_t* k, uint16_t* k_cmp, int B, int H_kv, int S_k,
                             hipStream_t stream);

hipError_t launch_select_blocks(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx,
                                float* blk_score, const AttnShape& s, hipStream_t stream);

// bytes of workspace the attention kernels need (V relayout + split partials)
size_t attn_workspace_bytes(const AttnShape& s);

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* blk_idx, uint16_t* out, float* lse,
                              const AttnShape& s, void* workspace, hipStream_t stream);

hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, const AttnShape& s, void* workspace,
                             hipStream_t stream);

// workspace of the sparse backward: D = <dO, O> per (token, head), then the
// selected-entry bitmap (one bit per KV head, block and query token)
size_t attn_bwd_workspace_bytes(const AttnShape& s);

hipError_t launch_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                                  const float* lse, const uint16_t* dout, const int32_t* blk_idx, uint16_t* dq,
                                  uint16_t* dk, uint16_t* dv, const AttnShape& s, float scale, void* workspace,
                                  hipStream_t stream);

}  // namespace infv2
