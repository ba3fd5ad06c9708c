/*
 * infv2.h — C ABI of the InfLLM-V2 block-sparse attention path for AMD
 * Instinct MI355X (gfx950): the forward (compression, block selection,
 * sparse and dense attention, the switch), the sparse backward, decode over a
 * paged cache, the approximate-LSE selection and the compressed-attention
 * branch with its mix.
 *
 * The method (pages: "Infllm V2 Dense Sparse Switchable Attention", skill
 * page; "InfLLM-V2: Dense-Sparse Switchable Attention for Seamless
 * Short-to-Long Adaptation", paper page; the InfLLM-V2 news summary):
 * keys are compressed into per-block means, every query token scores the
 * blocks with a per-head softmax over the compressed keys summed over its
 * GQA head group, picks the top-k blocks, and attends only to those blocks
 * plus the initial blocks and a causal sliding window of blocks.  Short
 * sequences take dense causal attention instead.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are contiguous, row-major, [B][H][S][D] (batch, heads, sequence,
 *    head dim), as in the shape docstrings of the skill page, Step 2.
 *    bf16 tensors are passed as raw 16-bit patterns (void*).
 *  - All tensor pointers are DEVICE pointers owned by the caller; every
 *    pointer must be 16-byte aligned (int32 length and table arrays: 4-byte).
 *    Outputs must not alias inputs, except where an entry point says so
 *    (the compressed branch may write its mix over the sparse output).
 *  - GQA: query head h reads KV head h / G with G = H_q / H_kv.
 *  - Query row r sits at absolute position i = (S_k - S_q) + r (bottom-right
 *    alignment; a single decode query is the last token of its cache).
 *  - Block j covers key positions [j*block_size, (j+1)*block_size);
 *    NB = ceil(S_k / block_size).
 *  - softmax_scale <= 0 selects 1/sqrt(D) (skill page, Step 1).
 *  - stream is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns; it never allocates device
 *    memory, never frees, never synchronises.  Device faults surface at the
 *    caller's next synchronisation.
 *  - Return value: INFV2_OK or an error code.  All argument checks run before
 *    any HIP call; on an error nothing is launched and outputs are untouched.
 *    Supported on the GPU: D = 128, block_size = 64, 1 <= G <= 16,
 *    0 <= topk <= 256, and at most 4064 key blocks (S_k <= 260096) for the
 *    block selection, the sparse forward and backward and the switch (2048
 *    for the one-query decode selection, infv2_decode_select), at most
 *    65535 (batch, kv head) pairs and B * H_kv * S_k <= 2^25 (the launch
 *    grids' limits); other values give INFV2_ERR_UNSUPPORTED.
 *  - The library keeps no state between calls; calls on distinct streams
 *    with distinct outputs and workspaces are independent.
 */
#ifndef INFV2_H
#define INFV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum infv2_status {
  INFV2_OK = 0,
  INFV2_ERR_INVALID = 1,      /* null/misaligned pointer, bad size or count */
  INFV2_ERR_UNSUPPORTED = 2,  /* valid, but outside what the kernels support */
  INFV2_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required  */
  INFV2_ERR_HIP = 4           /* the HIP runtime reported an error on launch */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* infv2_status_string(int status);

/* ABI version; bumped whenever a signature or a layout changes. */
int infv2_abi_version(void);

/*
 * Key compression (skill page, Step 2, compressed_attention: zero-pad to a
 * multiple of the block size, mean over each block's tokens).
 *   k      bf16 [B][H_kv][S_k][D]             (input)
 *   k_cmp  bf16 [B][H_kv][NB][D]              (output)
 * k_cmp[b,g,j,:] = bf16_RNE( sum_{t in block j, t < S_k} k[b,g,t,:] / block_size ).
 * The tail block is zero-padded: its divisor is block_size, not its length.
 * Sums are accumulated in fp64 and rounded once to bf16, nearest-even.
 */
int infv2_compress_k(const void* k, void* k_cmp,
                     int B, int H_kv, int S_k, int D, int block_size,
                     void* stream);

/*
 * Block selection: group-summed block scores and top-k (skill page,
 * Architecture Overview: the kernel sums log-sum-exp–normalised scores over
 * each head group; Step 2, selected_attention: top-k per query position; the
 * news summary, Technical Mechanism: the unit of selection is a block).
 *   q          bf16  [B][H_q][S_q][D]
 *   k_cmp      bf16  [B][H_kv][NB][D]      (from infv2_compress_k)
 *   blk_idx    int32 [B][H_kv][S_q][topk]  (output)
 *   blk_score  fp32  [B][H_kv][S_q][topk]  (optional output, may be NULL)
 * For query position i: nv = floor((i+1)/block_size) blocks are fully visible;
 * per head h of group g, z_hj = scale*<q_h, k_cmp_j>, p_hj = exp(z_hj -
 * logsumexp_{j<nv} z_hj) (exact log-sum-exp), sigma_j = sum_h p_hj.
 * Candidates are n_init <= j <= floor(i/block_size) - n_local; the
 * min(topk, #candidates) largest sigma are kept, equal sigma going to the
 * lower index.  Indices are written ascending, the rest of the row is -1;
 * blk_score holds sigma of each kept index (0 for padding).
 * Requires n_init >= 0, n_local >= 1.  No workspace is needed.
 */
int infv2_select_blocks(const void* q, const void* k_cmp,
                        int32_t* blk_idx, float* blk_score,
                        int B, int H_q, int H_kv, int S_q, int S_k, int D,
                        int block_size, int topk, int n_init, int n_local,
                        float softmax_scale, void* stream);

/*
 * Block selection with an approximate per-head log-sum-exp (skill page,
 * Architecture Overview: the two-pass selection kernel uses an approximate
 * LSE; the pages do not define it).  Reading: pass 1 evaluates each head's
 * softmax normaliser on every lse_stride-th visible compressed block only,
 * block R*x standing for the R = lse_stride blocks R*x .. R*x+R-1 (the last
 * group for its visible count):
 *   LSE_h ~ log sum_x min(R, nv - R*x) exp(scale q_h . k_cmp[R*x]).
 * Pass 2 and the top-k are those of infv2_select_blocks, so R = 1 gives
 * exactly its result.  Pass 1 streams 1/R of the compressed keys; the
 * selection can differ from the exact one (only through the per-head
 * normalisers: a common factor would not change it).  lse_stride: 1, 2, 4
 * or 8, else INFV2_ERR_UNSUPPORTED.  Layouts as infv2_select_blocks.
 */
int infv2_select_blocks_strided_lse(const void* q, const void* k_cmp,
                                    int32_t* blk_idx, float* blk_score,
                                    int B, int H_q, int H_kv, int S_q, int S_k, int D,
                                    int block_size, int topk, int n_init, int n_local,
                                    float softmax_scale, int lse_stride, void* stream);

/*
 * Block-sparse attention forward (news summary, Technical Mechanism:
 * attention computed only on the selected key-value blocks; skill page,
 * Step 2, sliding_attention, made causal and block-granular).
 *   q        bf16  [B][H_q][S_q][D]
 *   k, v     bf16  [B][H_kv][S_k][D]
 *   blk_idx  int32 [B][H_kv][S_q][topk]   entries in [0, NB) or -1 (ignored);
 *                                          duplicates and forced blocks are
 *                                          allowed and counted once
 *   out      bf16  [B][H_q][S_q][D]       (output)
 *   lse      fp32  [B][H_q][S_q]          (optional output, natural log)
 * Query position i attends keys t <= i of the blocks
 *   {0..n_init-1} U {qb-n_local+1 .. qb} U {selected},  qb = floor(i/block_size).
 * workspace: device memory of at least infv2_sparse_workspace_bytes(...)
 * bytes, 256-byte aligned; its contents on entry do not matter.  Long query
 * ranges need none (0 bytes).  For few query windows (decode) the block list
 * of a window is split over several workgroups whose fp32 partial results
 * (nsplit x B x H_q x S_q rows of 132 floats) are merged by a second kernel;
 * the split count depends only on B, H_kv, S_q and topk.
 */
size_t infv2_sparse_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k,
                                    int D, int block_size, int topk);
int infv2_sparse_attn_fwd(const void* q, const void* k, const void* v,
                          const int32_t* blk_idx, void* out, float* lse,
                          int B, int H_q, int H_kv, int S_q, int S_k, int D,
                          int block_size, int topk, int n_init, int n_local,
                          float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse attention backward (skill page, Step 5: Training and
 * Fine-tuning Procedure: the attention is trained by back-propagation).
 * Gradients of the attention of infv2_sparse_attn_fwd with respect to q, k
 * and v, over the same attended key sets; the block selection carries no
 * gradient.
 *   q, out, dout  bf16 [B][H_q][S_q][D]    (forward input, forward output,
 *                                           gradient of the output)
 *   k, v          bf16 [B][H_kv][S_k][D]
 *   lse           fp32 [B][H_q][S_q]       (required: the forward's natural-log
 *                                           log-sum-exp)
 *   blk_idx       int32 [B][H_kv][S_q][topk] (as for the forward)
 *   dq            bf16 [B][H_q][S_q][D]    (output)
 *   dk, dv        bf16 [B][H_kv][S_k][D]   (output, overwritten; keys no query
 *                                           attends get 0)
 * With P the softmax weights, D = <dout, out> per (token, head) and
 * dS = P * (dout v^T - D):  dq = scale dS k,  dk = scale sum dS^T q,
 * dv = sum P^T dout, the sums over every (token, head of the group) that
 * attends the key.  Accumulation is fp32, each output rounded once to bf16;
 * the result does not depend on scheduling (no atomics on gradients).
 * workspace: at least infv2_sparse_bwd_workspace_bytes(...) bytes, 256-byte
 * aligned, contents on entry irrelevant (4 bytes per query row and head, one
 * bit per KV head, block and query token, and from 4096 queries the fp32
 * partial key and value gradients of each token piece: 64 KB per KV head, key
 * block and piece, 2 pieces from 4096 queries and 16 from 12288, so 1.07 GB
 * for 2 KV heads at 32768 keys).  S_q = 0 needs none and writes zero dk, dv.
 */
size_t infv2_sparse_bwd_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k,
                                        int D, int block_size, int topk);
int infv2_sparse_attn_bwd(const void* q, const void* k, const void* v,
                          const void* out, const float* lse, const void* dout,
                          const int32_t* blk_idx, void* dq, void* dk, void* dv,
                          int B, int H_q, int H_kv, int S_q, int S_k, int D,
                          int block_size, int topk, int n_init, int n_local,
                          float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense attention forward (skill page, Step 1: Dense Attention Layer
 * Foundation), GQA, causal (keys t <= i) or not (all S_k keys).
 * Same tensor layouts as infv2_sparse_attn_fwd; workspace of at least
 * infv2_dense_workspace_bytes(...) bytes, 256-byte aligned.
 */
size_t infv2_dense_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k, int D);
int infv2_dense_attn_fwd(const void* q, const void* k, const void* v,
                         void* out, float* lse,
                         int B, int H_q, int H_kv, int S_q, int S_k, int D,
                         float softmax_scale, int causal,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * The dense/sparse switch (skill page, Step 3: a sequence no longer than the
 * threshold runs dense; paper page, Abstract: dense for short inputs, sparse
 * for long ones).  Causal.  If S_k <= switch_len: infv2_dense_attn_fwd.
 * Otherwise compress -> select -> sparse; k_cmp, blk_idx and the sparse
 * workspace are carved from `workspace`.
 * blk_idx_out (optional, may be NULL) receives the selection
 * int32 [B][H_kv][S_q][topk] when the sparse path runs.
 */
size_t infv2_attn_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k,
                                  int D, int block_size, int topk, int switch_len);
/*
 * The path infv2_attn_fwd (and infv2_attn_fwd_noalloc) takes for S_k keys
 * under switch_len: INFV2_PATH_DENSE or INFV2_PATH_SPARSE.  Pure host
 * function, no HIP call; the one place the switch rule is written.
 */
enum infv2_path { INFV2_PATH_SPARSE = 0, INFV2_PATH_DENSE = 1 };
int infv2_attn_path(int S_k, int switch_len);
int infv2_attn_fwd(const void* q, const void* k, const void* v,
                   void* out, float* lse, int32_t* blk_idx_out,
                   int B, int H_q, int H_kv, int S_q, int S_k, int D,
                   int block_size, int topk, int n_init, int n_local,
                   float softmax_scale, int switch_len,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * infv2_attn_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as infv2_attn_fwd (blk_idx_out optional), but
 * the workspace is a fixed array of INFV2_NOALLOC_SCRATCH_BYTES (32 MiB) in
 * the library's device memory, one per GPU, held until the process ends;
 * the call allocates nothing.  A shape whose infv2_attn_workspace_bytes
 * exceeds it returns INFV2_ERR_WORKSPACE before any HIP call (32 MiB covers
 * the switch up to 32768 tokens with 2 KV heads and top-64).  The stream must
 * belong to the current device.  Every call on one GPU uses that GPU's one
 * array: calls that overlap on a GPU (other streams, other threads) race and
 * give unspecified results; calls in stream order do not.  Nothing in the
 * array needs to start at zero (a call writes every byte it reads).
 */
#define INFV2_NOALLOC_SCRATCH_BYTES (32u << 20)
int infv2_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                           void* out, float* lse, int32_t* blk_idx_out,
                           int B, int H_q, int H_kv, int S_q, int S_k, int D,
                           int block_size, int topk, int n_init, int n_local,
                           float softmax_scale, int switch_len, void* stream);

/*
 * Decode over a paged, variable-length KV cache (news summary, Performance
 * Evaluation: the method also speeds up decoding).  One new query token per
 * sequence; sequence b holds seqlens[b] keys and its query is the last of
 * them (key position seqlens[b] - 1), so the three calls below give, per
 * sequence, exactly what infv2_compress_k, infv2_select_blocks and
 * infv2_sparse_attn_fwd give for S_q = 1 on that sequence's contiguous keys.
 *   k_pages, v_pages  bf16 [num_pages][H_kv][block_size][D]: a page is one
 *                     key block of every KV head
 *   block_table       int32 [B][max_blocks]: page of logical block j of
 *                     sequence b, in [0, num_pages)
 *   seqlens           int32 [B]: keys of sequence b, in [1, max_blocks *
 *                     block_size]
 *   k_cmp             bf16 [B][H_kv][max_blocks][D]: compressed keys of the
 *                     complete blocks (j < floor(seqlens[b] / block_size);
 *                     other rows are not read)
 *   q, out            bf16 [B][H_q][D];  lse fp32 [B][H_q] (optional)
 *   blk_idx           int32 [B][H_kv][topk]
 * Lengths, table entries and page ids live in device memory and are not
 * checked on the host: out-of-range values are clamped into range on the
 * GPU (no out-of-bounds access), with unspecified results.
 * A sequence with no more than n_init + n_local + topk blocks attends every
 * one of its keys, i.e. runs dense: no separate switch is needed.
 */

/* Compressed keys of the blocks that became complete when each sequence
 * grew from old_lens[b] to new_lens[b] keys: blocks floor(old/bs) ..
 * floor(new/bs) - 1, at most max_new_blocks per sequence (1 per generated
 * token; floor(max_len / bs) to fill a cache from scratch, old_lens = 0).
 * Other rows of k_cmp are left untouched. */
int infv2_decode_compress_append(const void* k_pages, const int32_t* block_table,
                                 const int32_t* old_lens, const int32_t* new_lens,
                                 void* k_cmp, int B, int H_kv, int D, int block_size,
                                 int max_blocks, int num_pages, int max_new_blocks,
                                 void* stream);

/* Block selection of each sequence's query (as infv2_select_blocks). */
int infv2_decode_select(const void* q, const void* k_cmp, const int32_t* seqlens,
                        int32_t* blk_idx, float* blk_score,
                        int B, int H_q, int H_kv, int D, int block_size,
                        int max_blocks, int topk, int n_init, int n_local,
                        float softmax_scale, void* stream);

/* Block-sparse attention of each sequence's query over its paged keys (as
 * infv2_sparse_attn_fwd); workspace of at least
 * infv2_decode_attn_workspace_bytes(...) bytes, 256-byte aligned, for the
 * split partials (nsplit x B x H_q rows of 132 floats). */
size_t infv2_decode_attn_workspace_bytes(int B, int H_q, int H_kv, int D, int block_size,
                                         int max_blocks, int topk);
int infv2_decode_attn(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* seqlens,
                      const int32_t* blk_idx, void* out, float* lse,
                      int B, int H_q, int H_kv, int D, int block_size,
                      int max_blocks, int num_pages, int topk, int n_init, int n_local,
                      float softmax_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/* infv2_decode_select followed by infv2_decode_attn, in one launch (plus the
 * merge of the split partials): the same blk_idx and blk_score (blk_score
 * may be null), out and lse (may be null), bit for bit.  Each of the
 * workgroups that share a sequence's KV head repeats that head's selection
 * on its own CU and attends its share of the selected blocks at once, so
 * the selection's result never goes through device memory on its way to the
 * attention.  Same arguments and limits as those two calls (max_blocks <=
 * 2048); workspace as for infv2_decode_attn. */
int infv2_decode_select_attn(const void* q, const void* k_cmp, const void* k_pages,
                             const void* v_pages, const int32_t* block_table,
                             const int32_t* seqlens, int32_t* blk_idx, float* blk_score,
                             void* out, float* lse,
                             int B, int H_q, int H_kv, int D, int block_size,
                             int max_blocks, int num_pages, int topk, int n_init, int n_local,
                             float softmax_scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Compressed-attention branch and the mix of patterns (skill page, Step 2,
 * compressed_attention: queries attend block means of the keys and values;
 * Step 3: the sparse context is a weighted sum of the pattern outputs).
 * Readings: the branch is causal like block scoring - the query at position
 * i (bottom-right aligned, i = S_k - S_q + r) attends the compressed keys of
 * the nv = floor((i+1)/block_size) blocks wholly at or before it; the mixing
 * coefficients are arguments (the page learns them; this library has no
 * parameters); the block-sparse output (selected, initial and window blocks
 * in one softmax) is one pattern, this branch the other.
 *   q                bf16 [B][H_q][S_q][D]
 *   k_cmp, v_cmp     bf16 [B][H_kv][NB][D], NB = ceil(S_k/block_size), from
 *                    infv2_compress_k and infv2_compress_v
 *   o_sparse         bf16 [B][H_q][S_q][D] (optional, may be NULL): e.g.
 *                    the output of infv2_sparse_attn_fwd
 *   out              bf16 [B][H_q][S_q][D]; may be o_sparse itself
 *   lse              fp32 [B][H_q][S_q] (optional): the branch's own natural
 *                    log-sum-exp, -inf where nv = 0
 * out = w_cmp * softmax_{j<nv}(scale q.k_cmp_j) v_cmp  [+ w_sparse * o_sparse]
 * A query with nv = 0 (position below block_size - 1) contributes a zero
 * branch output.  w_sparse, w_cmp must be finite (else INFV2_ERR_INVALID).
 * No workspace.  Errors as for infv2_sparse_attn_fwd.
 */
int infv2_compress_v(const void* v, void* v_cmp,
                     int B, int H_kv, int S_k, int D, int block_size,
                     void* stream);
int infv2_compressed_attn_fwd(const void* q, const void* k_cmp, const void* v_cmp,
                              const void* o_sparse, void* out, float* lse,
                              int B, int H_q, int H_kv, int S_q, int S_k, int D,
                              int block_size, float softmax_scale,
                              float w_sparse, float w_cmp, void* stream);

/* The block-sparse attention and the compressed branch in one call:
 *   out = w_sparse * infv2_sparse_attn_fwd(...) + w_cmp * compressed branch
 * with the arguments and layouts of infv2_sparse_attn_fwd plus k_cmp, v_cmp
 * of infv2_compressed_attn_fwd; lse is the sparse attention's.  One launch
 * streams each query window's compressed groups and then its selected blocks
 * through the same pipeline; the branch passes through out (rounded once to
 * bf16) before the sparse part is added.  Shapes whose block lists are split
 * over several workgroups (few query windows, as in decode) run the two
 * calls one after the other instead, with the same result definition.
 * Workspace: infv2_sparse_workspace_bytes(...). */
int infv2_mixed_attn_fwd(const void* q, const void* k, const void* v,
                         const int32_t* blk_idx, const void* k_cmp, const void* v_cmp,
                         void* out, float* lse,
                         int B, int H_q, int H_kv, int S_q, int S_k, int D,
                         int block_size, int topk, int n_init, int n_local,
                         float softmax_scale, float w_sparse, float w_cmp,
                         void* workspace, size_t workspace_bytes, void* stream);

/* The compressed-attention branch of each decode query (as
 * infv2_compressed_attn_fwd for S_q = 1 on that sequence): k_cmp, v_cmp
 * [B][H_kv][max_blocks][D] from infv2_decode_compress_append on the key and
 * on the value pages; q, o_sparse, out bf16 [B][H_q][D]; lse fp32 [B][H_q].
 * Lengths are clamped on the GPU as for the other decode calls. */
int infv2_decode_compressed_attn(const void* q, const void* k_cmp, const void* v_cmp,
                                 const int32_t* seqlens, const void* o_sparse,
                                 void* out, float* lse,
                                 int B, int H_q, int H_kv, int D, int block_size,
                                 int max_blocks, float softmax_scale,
                                 float w_sparse, float w_cmp, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INFV2_H */
