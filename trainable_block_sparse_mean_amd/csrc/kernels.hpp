// Internal launch functions of the gfx950 kernels (called by api.hip after
// argument validation).  Shapes here are already checked: D = 128,
// block size 64, 1 <= G <= 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace infv2 {

// Key blocks the sparse kernels take (S_k <= 260096): the 128 KB K/V ring
// and the window's union list (8 bytes per block, plus 16) fit in the 160 KB
// of LDS of a workgroup.
constexpr int kMaxSparseBlocks = 4064;
// Key blocks of a decode sequence (one query) the decode selection takes: 16
// waves of 8 tiles of 16 blocks hold every score in registers.
constexpr int kMaxDecodeSelectBlocks = 2048;

struct AttnShape {
  int B, H_q, H_kv, S_q, S_k, G, NB;
  int topk, n_init, n_local;
  float scale_log2;  // softmax scale * log2(e)
  int causal;
  int nsplit;        // sparse: workgroups sharing one window's block list (1 = no split)
  // A paged, variable-length key cache (decode); both null for one key
  // length S_k and contiguous [B][H_kv][S_k][D] K/V.
  //   seqlens[b]: keys of sequence b, 1 .. NB * 64 (its queries end at key
  //     seqlens[b] - 1); NB is then the per-sequence block capacity, the row
  //     stride of block_table and of the compressed keys.
  //   block_table[b * NB + j]: the page holding logical block j of sequence
  //     b, 0 .. num_pages - 1; a page is one 64-key block of every KV head,
  //     [H_kv][64][D].
  const int* seqlens;
  const int* block_table;
  int num_pages;
};

// keys of sequence b (the uniform S_k without a length table), clamped to
// the block capacity so that a bad length cannot address past the table
__device__ __forceinline__ int seq_keys(const AttnShape& s, int b) {
  return s.seqlens ? min(max(s.seqlens[b], 1), s.NB * 64) : s.S_k;
}

// first row of block j of (batch b, KV head g) in a paged cache of
// [page][H_kv][64][128] rows (page ids clamped into range, so that a bad
// table cannot address past the pages)
__device__ __forceinline__ size_t page_rows(const AttnShape& s, int b, int g, int j) {
  const int page = min(max(s.block_table[static_cast<size_t>(b) * s.NB + j], 0), s.num_pages - 1);
  return (static_cast<size_t>(page) * s.H_kv + g) * 64 * 128;
}

// Split-KV partials of the sparse kernel, in the workspace: for split s and
// query row (b, h, r), 128 unnormalised fp32 output values relative to the
// split's running max, then that max (log2 units) and the row sum (two
// padding floats keep rows 16-byte aligned).
constexpr int kPartFloats = 132;  // 128 + m + l, padded to 16 bytes

// number of splits the sparse kernel uses for a shape (1 for long queries)
int sparse_splits(int B, int H_kv, int S_q, int topk);

hipError_t launch_compress_k(const uint16_t* k, uint16_t* k_cmp, int B, int H_kv, int S_k,
                             hipStream_t stream);

// compressed keys of the blocks of a paged cache that became complete when
// sequence b grew from old_len[b] to new_len[b] keys (at most max_new per
// sequence); k_cmp is [B][H_kv][NB][D]
hipError_t launch_compress_append(const uint16_t* k_pages, const AttnShape& s, const int* old_len,
                                  uint16_t* k_cmp, int max_new, hipStream_t stream);

// lse_stride 1: exact pass-1 log-sum-exp; 2, 4 or 8: the strided approximation
hipError_t launch_select_blocks(const uint16_t* q, const uint16_t* k_cmp, int32_t* blk_idx,
                                float* blk_score, const AttnShape& s, hipStream_t stream, int lse_stride = 1);

// bytes of workspace the sparse forward needs: the split-KV partials (0 when
// a shape runs unsplit)
size_t attn_workspace_bytes(const AttnShape& s);

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* blk_idx, uint16_t* out, float* lse,
                              const AttnShape& s, void* workspace, hipStream_t stream);

// merge the split-KV partials of the sparse kernels (s.nsplit splits) into
// out and lse
hipError_t launch_combine_splits(const float* part, uint16_t* out, float* lse, const AttnShape& s,
                                 hipStream_t stream);
// Decode (one query per sequence and KV head, S_q = 1, at most 2048 key
// blocks): the exact selection and the block-sparse attention in one launch
// (plus the merge of the split partials); blk_idx [B][H_kv][1][topk] (and
// blk_score, if not null) receive the selection.
hipError_t launch_decode_select_attn(const uint16_t* q, const uint16_t* k_cmp, const uint16_t* k, const uint16_t* v,
                                     int32_t* blk_idx, float* blk_score, uint16_t* out, float* lse,
                                     const AttnShape& s, void* workspace, hipStream_t stream);
hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, const AttnShape& s, void* workspace,
                             hipStream_t stream);

// Compressed-attention branch over k_cmp / v_cmp [B][H_kv][NB][D] (NB = s.NB
// compressed rows per KV head): out = w_cmp * O_cmp (+ w_sparse * o_sparse
// when o_sparse is not null; out may equal o_sparse); lse (optional) is the
// branch's own log-sum-exp, -inf for a query that sees no block.
hipError_t launch_compressed_attn(const uint16_t* q, const uint16_t* k_cmp, const uint16_t* v_cmp,
                                  const uint16_t* o_sparse, uint16_t* out, float* lse, const AttnShape& s,
                                  float w_sparse, float w_cmp, hipStream_t stream);

// The block-sparse attention and the compressed branch in one launch: out =
// w_sparse * O_sparse + w_cmp * O_cmp (the branch goes through out in bf16 on
// its way); lse is the sparse attention's.  Shapes that split the block list
// (few query windows) run the two kernels one after the other instead.
hipError_t launch_mixed_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* blk_idx,
                             const uint16_t* k_cmp, const uint16_t* v_cmp, uint16_t* out, float* lse,
                             const AttnShape& s, float w_sparse, float w_cmp, void* workspace, hipStream_t stream);

// workspace of the sparse backward: D = <dO, O> per (token, head), then the
// selected-entry bitmap (one bit per KV head, block and query token)
size_t attn_bwd_workspace_bytes(const AttnShape& s);

hipError_t launch_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                                  const float* lse, const uint16_t* dout, const int32_t* blk_idx, uint16_t* dq,
                                  uint16_t* dk, uint16_t* dv, const AttnShape& s, float scale, void* workspace,
                                  hipStream_t stream);

}  // namespace infv2
