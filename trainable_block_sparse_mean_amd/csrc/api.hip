// C ABI of the InfLLM-V2 sparse attention path (declared in include/infv2.h):
// argument validation, workspace sizing and kernel dispatch.  Every check runs
// before the first HIP call, so an invalid call launches nothing.
#include <math.h>

#include <mutex>

#include "infv2.h"
#include "common.hpp"
#include "kernels.hpp"

using infv2::AttnShape;

namespace {

constexpr int kAbiVersion = 1;
constexpr int kMaxTopk = 256;
// Selection keeps each token's block scores in LDS: up to 4064 blocks for
// prefill queries (as many as the sparse kernels take), 2048 for one-query
// decode selection (a wave holds at most 8 tiles of 16 blocks).
constexpr int kMaxSelectBlocks = infv2::kMaxSparseBlocks;
using infv2::kMaxDecodeSelectBlocks;
// the sparse kernels keep a member mask and a list entry (8 bytes) per key
// block in LDS beside the 128 KB K/V ring (kernels.hpp)
using infv2::kMaxSparseBlocks;

// Launch-grid limits: the kernels put the (batch, kv head) pairs in gridDim.y
// (at most 65535), and a grid spans about 64 work-items per key and kv head,
// which must stay below 2^32.
constexpr long long kMaxHeadRows = 65535;
constexpr long long kMaxHeadKeys = 1LL << 25;

bool grid_fits(long long B, long long H_kv, long long S_k) {
  return B * H_kv <= kMaxHeadRows && B * H_kv * S_k <= kMaxHeadKeys;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int num_blocks(int S_k, int block_size) { return (S_k + block_size - 1) / block_size; }

// shape checks shared by every attention-type entry point
int check_shape(int B, int H_q, int H_kv, int S_q, int S_k, int D) {
  if (B < 0 || H_q < 1 || H_kv < 1 || S_q < 0 || S_k < 0 || D < 1) return INFV2_ERR_INVALID;
  if (H_q % H_kv != 0 || S_q > S_k) return INFV2_ERR_INVALID;
  if (D != infv2::kD) return INFV2_ERR_UNSUPPORTED;
  if (H_q / H_kv > infv2::kMaxG) return INFV2_ERR_UNSUPPORTED;
  // element offsets are computed in 64 bits; keep sequence indices in int range
  if (static_cast<long long>(S_k) * D >= (1LL << 31)) return INFV2_ERR_UNSUPPORTED;
  if (!grid_fits(B, H_kv, S_k)) return INFV2_ERR_UNSUPPORTED;
  return INFV2_OK;
}

int check_sparse_params(int block_size, int topk, int n_init, int n_local) {
  if (block_size < 1 || topk < 0 || n_init < 0 || n_local < 1) return INFV2_ERR_INVALID;
  if (block_size != infv2::kBS || topk > kMaxTopk) return INFV2_ERR_UNSUPPORTED;
  return INFV2_OK;
}

bool tensor_ok(const void* p) { return p != nullptr && aligned(p, 16); }

float scale_log2(float softmax_scale, int D) {
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf(static_cast<float>(D));
  return sc * infv2::kLog2e;
}

AttnShape make_shape(int B, int H_q, int H_kv, int S_q, int S_k, int block_size, int topk,
                     int n_init, int n_local, float sl2, int causal) {
  AttnShape s;
  s.B = B;
  s.H_q = H_q;
  s.H_kv = H_kv;
  s.S_q = S_q;
  s.S_k = S_k;
  s.G = H_q / H_kv;
  s.NB = num_blocks(S_k, block_size);
  s.topk = topk;
  s.n_init = n_init;
  s.n_local = n_local;
  s.scale_log2 = sl2;
  s.causal = causal;
  s.nsplit = 1;
  s.seqlens = nullptr;
  s.block_table = nullptr;
  s.num_pages = 0;
  return s;
}

int hip_status(hipError_t e) { return e == hipSuccess ? INFV2_OK : INFV2_ERR_HIP; }

// ---- decode over a paged, variable-length cache -----------------------------
int check_decode(int B, int H_q, int H_kv, int D, int block_size, int max_blocks) {
  if (B < 0 || H_q < 1 || H_kv < 1 || D < 1 || block_size < 1 || max_blocks < 1) return INFV2_ERR_INVALID;
  if (H_q % H_kv != 0) return INFV2_ERR_INVALID;
  if (D != infv2::kD || block_size != infv2::kBS) return INFV2_ERR_UNSUPPORTED;
  if (H_q / H_kv > infv2::kMaxG) return INFV2_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_blocks) * block_size * D >= (1LL << 31)) return INFV2_ERR_UNSUPPORTED;
  if (!grid_fits(B, H_kv, static_cast<long long>(max_blocks) * block_size)) return INFV2_ERR_UNSUPPORTED;
  return INFV2_OK;
}

bool ints_ok(const void* p) { return p != nullptr && aligned(p, 4); }

// one query per sequence (S_q = 1) at key seqlens[b] - 1 of a cache of
// max_blocks blocks per sequence
AttnShape decode_shape(int B, int H_q, int H_kv, int max_blocks, int topk, int n_init, int n_local, float sl2,
                       const int32_t* seqlens, const int32_t* block_table, int num_pages) {
  AttnShape s = make_shape(B, H_q, H_kv, 1, max_blocks * infv2::kBS, infv2::kBS, topk, n_init, n_local, sl2, 1);
  s.seqlens = seqlens;
  s.block_table = block_table;
  s.num_pages = num_pages;
  return s;
}

size_t sparse_ws(int B, int H_q, int H_kv, int S_q, int S_k, int block_size, int topk) {
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, 0, 1, 1.f, 1);
  return round_up(infv2::attn_workspace_bytes(s), 256);
}

}  // namespace

extern "C" {

const char* infv2_status_string(int status) {
  switch (status) {
    case INFV2_OK: return "ok";
    case INFV2_ERR_INVALID: return "invalid argument";
    case INFV2_ERR_UNSUPPORTED: return "unsupported configuration";
    case INFV2_ERR_WORKSPACE: return "workspace missing or too small";
    case INFV2_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int infv2_abi_version(void) { return kAbiVersion; }

int infv2_compress_k(const void* k, void* k_cmp, int B, int H_kv, int S_k, int D, int block_size,
                     void* stream) {
  if (B < 0 || H_kv < 1 || S_k < 0 || D < 1 || block_size < 1) return INFV2_ERR_INVALID;
  if (D != infv2::kD || block_size != infv2::kBS) return INFV2_ERR_UNSUPPORTED;
  if (static_cast<long long>(S_k) * D >= (1LL << 31)) return INFV2_ERR_UNSUPPORTED;
  if (!grid_fits(B, H_kv, S_k)) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_k == 0) return INFV2_OK;
  if (!tensor_ok(k) || !tensor_ok(k_cmp)) return INFV2_ERR_INVALID;
  return hip_status(infv2::launch_compress_k(static_cast<const uint16_t*>(k), static_cast<uint16_t*>(k_cmp),
                                             B, H_kv, S_k, static_cast<hipStream_t>(stream)));
}

int infv2_select_blocks(const void* q, const void* k_cmp, int32_t* blk_idx, float* blk_score, int B,
                        int H_q, int H_kv, int S_q, int S_k, int D, int block_size, int topk,
                        int n_init, int n_local, float softmax_scale, void* stream) {
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (num_blocks(S_k, block_size) > kMaxSelectBlocks) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_q == 0 || topk == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k_cmp) || !tensor_ok(blk_idx)) return INFV2_ERR_INVALID;
  if (blk_score && !aligned(blk_score, 16)) return INFV2_ERR_INVALID;
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, n_init, n_local,
                                 scale_log2(softmax_scale, D), 1);
  return hip_status(infv2::launch_select_blocks(static_cast<const uint16_t*>(q),
                                                static_cast<const uint16_t*>(k_cmp), blk_idx, blk_score,
                                                s, static_cast<hipStream_t>(stream)));
}

int infv2_select_blocks_strided_lse(const void* q, const void* k_cmp, int32_t* blk_idx, float* blk_score, int B,
                                    int H_q, int H_kv, int S_q, int S_k, int D, int block_size, int topk,
                                    int n_init, int n_local, float softmax_scale, int lse_stride, void* stream) {
  if (lse_stride != 1 && lse_stride != 2 && lse_stride != 4 && lse_stride != 8) return INFV2_ERR_UNSUPPORTED;
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (num_blocks(S_k, block_size) > kMaxSelectBlocks) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_q == 0 || topk == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k_cmp) || !tensor_ok(blk_idx)) return INFV2_ERR_INVALID;
  if (blk_score && !aligned(blk_score, 16)) return INFV2_ERR_INVALID;
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, n_init, n_local,
                                 scale_log2(softmax_scale, D), 1);
  return hip_status(infv2::launch_select_blocks(static_cast<const uint16_t*>(q),
                                                static_cast<const uint16_t*>(k_cmp), blk_idx, blk_score, s,
                                                static_cast<hipStream_t>(stream), lse_stride));
}

size_t infv2_sparse_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k, int D, int block_size,
                                    int topk) {
  if (check_shape(B, H_q, H_kv, S_q, S_k, D) != INFV2_OK || block_size != infv2::kBS || topk < 0) return 0;
  return sparse_ws(B, H_q, H_kv, S_q, S_k, block_size, topk);
}

int infv2_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* blk_idx, void* out,
                          float* lse, int B, int H_q, int H_kv, int S_q, int S_k, int D, int block_size,
                          int topk, int n_init, int n_local, float softmax_scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (num_blocks(S_k, block_size) > kMaxSparseBlocks) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_q == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out)) return INFV2_ERR_INVALID;
  if (topk > 0 && !tensor_ok(blk_idx)) return INFV2_ERR_INVALID;
  if (lse && !aligned(lse, 16)) return INFV2_ERR_INVALID;
  const size_t need = sparse_ws(B, H_q, H_kv, S_q, S_k, block_size, topk);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return INFV2_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return INFV2_ERR_INVALID;
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, n_init, n_local,
                                 scale_log2(softmax_scale, D), 1);
  return hip_status(infv2::launch_sparse_attn(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      blk_idx, static_cast<uint16_t*>(out), lse, s, workspace, static_cast<hipStream_t>(stream)));
}

size_t infv2_sparse_bwd_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k, int D, int block_size,
                                        int topk) {
  if (check_shape(B, H_q, H_kv, S_q, S_k, D) != INFV2_OK) return 0;
  if (check_sparse_params(block_size, topk, 0, 1) != INFV2_OK) return 0;
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, 0, 1, 1.f, 1);
  return round_up(infv2::attn_bwd_workspace_bytes(s), 256);
}

int infv2_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                          const void* dout, const int32_t* blk_idx, void* dq, void* dk, void* dv, int B, int H_q,
                          int H_kv, int S_q, int S_k, int D, int block_size, int topk, int n_init, int n_local,
                          float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (num_blocks(S_k, block_size) > kMaxSparseBlocks) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_k == 0) return INFV2_OK;  // no key: nothing to write
  if (!tensor_ok(dk) || !tensor_ok(dv)) return INFV2_ERR_INVALID;
  if (S_q > 0) {
    if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out) || !tensor_ok(dout) ||
        !tensor_ok(dq) || !tensor_ok(lse))
      return INFV2_ERR_INVALID;
    if (topk > 0 && !tensor_ok(blk_idx)) return INFV2_ERR_INVALID;
    const size_t need = infv2_sparse_bwd_workspace_bytes(B, H_q, H_kv, S_q, S_k, D, block_size, topk);
    if (workspace == nullptr || workspace_bytes < need) return INFV2_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return INFV2_ERR_INVALID;
  }
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf(static_cast<float>(D));
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, n_init, n_local,
                                 sc * infv2::kLog2e, 1);
  return hip_status(infv2::launch_sparse_attn_bwd(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<const uint16_t*>(out), lse, static_cast<const uint16_t*>(dout), blk_idx,
      static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), s, sc, workspace,
      static_cast<hipStream_t>(stream)));
}

size_t infv2_dense_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k, int D) {
  if (check_shape(B, H_q, H_kv, S_q, S_k, D) != INFV2_OK) return 0;
  return sparse_ws(B, H_q, H_kv, S_q, S_k, infv2::kBS, 0);
}

int infv2_dense_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                         int H_q, int H_kv, int S_q, int S_k, int D, float softmax_scale, int causal,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  if (causal != 0 && causal != 1) return INFV2_ERR_INVALID;
  if (B == 0 || S_q == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out)) return INFV2_ERR_INVALID;
  if (lse && !aligned(lse, 16)) return INFV2_ERR_INVALID;
  const size_t need = sparse_ws(B, H_q, H_kv, S_q, S_k, infv2::kBS, 0);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return INFV2_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return INFV2_ERR_INVALID;
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, infv2::kBS, 0, 0, 1,
                                 scale_log2(softmax_scale, D), causal);
  return hip_status(infv2::launch_dense_attn(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                             static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse,
                                             s, workspace, static_cast<hipStream_t>(stream)));
}

int infv2_attn_path(int S_k, int switch_len) {
  return S_k <= switch_len ? INFV2_PATH_DENSE : INFV2_PATH_SPARSE;
}

size_t infv2_attn_workspace_bytes(int B, int H_q, int H_kv, int S_q, int S_k, int D, int block_size, int topk,
                                  int switch_len) {
  if (check_shape(B, H_q, H_kv, S_q, S_k, D) != INFV2_OK || block_size != infv2::kBS || topk < 0) return 0;
  if (infv2_attn_path(S_k, switch_len) == INFV2_PATH_DENSE) return infv2_dense_workspace_bytes(B, H_q, H_kv, S_q, S_k, D);
  const size_t kc = round_up(static_cast<size_t>(B) * H_kv * num_blocks(S_k, block_size) * D * 2, 256);
  const size_t idx = round_up(static_cast<size_t>(B) * H_kv * S_q * topk * 4, 256);
  return kc + idx + sparse_ws(B, H_q, H_kv, S_q, S_k, block_size, topk);
}

int infv2_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int32_t* blk_idx_out,
                   int B, int H_q, int H_kv, int S_q, int S_k, int D, int block_size, int topk, int n_init,
                   int n_local, float softmax_scale, int switch_len, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (infv2_attn_path(S_k, switch_len) == INFV2_PATH_DENSE)
    return infv2_dense_attn_fwd(q, k, v, out, lse, B, H_q, H_kv, S_q, S_k, D, softmax_scale, 1, workspace,
                                workspace_bytes, stream);
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (num_blocks(S_k, block_size) > kMaxSelectBlocks) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_q == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out)) return INFV2_ERR_INVALID;
  if (lse && !aligned(lse, 16)) return INFV2_ERR_INVALID;
  if (blk_idx_out && !aligned(blk_idx_out, 16)) return INFV2_ERR_INVALID;
  const size_t need = infv2_attn_workspace_bytes(B, H_q, H_kv, S_q, S_k, D, block_size, topk, switch_len);
  if (workspace == nullptr || workspace_bytes < need) return INFV2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return INFV2_ERR_INVALID;

  char* ws = static_cast<char*>(workspace);
  const size_t kc_bytes = round_up(static_cast<size_t>(B) * H_kv * num_blocks(S_k, block_size) * D * 2, 256);
  const size_t idx_bytes = round_up(static_cast<size_t>(B) * H_kv * S_q * topk * 4, 256);
  void* k_cmp = ws;
  int32_t* idx = blk_idx_out ? blk_idx_out : reinterpret_cast<int32_t*>(ws + kc_bytes);
  void* rest = ws + kc_bytes + idx_bytes;
  const size_t rest_bytes = workspace_bytes - kc_bytes - idx_bytes;

  st = infv2_compress_k(k, k_cmp, B, H_kv, S_k, D, block_size, stream);
  if (st != INFV2_OK) return st;
  if (S_q == 1 && topk > 0 && num_blocks(S_k, block_size) <= kMaxDecodeSelectBlocks) {
    // one query row per KV head (decode): selection and attention in one
    // launch, the same results as the two calls below
    const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, n_init, n_local,
                                   scale_log2(softmax_scale, D), 1);
    return hip_status(infv2::launch_decode_select_attn(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cmp), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), idx, nullptr, static_cast<uint16_t*>(out), lse, s, rest,
        static_cast<hipStream_t>(stream)));
  }
  if (topk > 0) {
    st = infv2_select_blocks(q, k_cmp, idx, nullptr, B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init,
                             n_local, softmax_scale, stream);
    if (st != INFV2_OK) return st;
  }
  return infv2_sparse_attn_fwd(q, k, v, idx, out, lse, B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init,
                               n_local, softmax_scale, rest, rest_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of infv2_attn_fwd_noalloc: the switch's workspace (compressed keys,
// block indices, split-KV partials), carved as in infv2_attn_fwd.  A file-scope
// device array, so the library never allocates it; each GPU the library runs on
// holds its own copy until the process ends.  Host code never takes the
// array's name as an address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = INFV2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's scratch (looked up on its first use)
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return INFV2_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return INFV2_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return INFV2_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return INFV2_OK;
}

}  // namespace

extern "C" {

int infv2_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                           int32_t* blk_idx_out, int B, int H_q, int H_kv, int S_q, int S_k, int D, int block_size,
                           int topk, int n_init, int n_local, float softmax_scale, int switch_len, void* stream) {
  // the argument checks of infv2_attn_fwd, then the size check, before any HIP call
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  if (infv2_attn_path(S_k, switch_len) == INFV2_PATH_SPARSE) {
    st = check_sparse_params(block_size, topk, n_init, n_local);
    if (st != INFV2_OK) return st;
    if (num_blocks(S_k, block_size) > kMaxSelectBlocks) return INFV2_ERR_UNSUPPORTED;
  }
  if (B == 0 || S_q == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out)) return INFV2_ERR_INVALID;
  if (lse && !aligned(lse, 16)) return INFV2_ERR_INVALID;
  if (blk_idx_out && !aligned(blk_idx_out, 16)) return INFV2_ERR_INVALID;
  const size_t need = infv2_attn_workspace_bytes(B, H_q, H_kv, S_q, S_k, D, block_size, topk, switch_len);
  if (need > kNoAllocScratchBytes) return INFV2_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(&ws);
    if (st != INFV2_OK) return st;
  }
  // every byte of the scratch a call reads was written earlier in the same
  // call (compressed keys, selected blocks, split partials): nothing is cleared
  return infv2_attn_fwd(q, k, v, out, lse, blk_idx_out, B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init,
                        n_local, softmax_scale, switch_len, ws, need > 0 ? kNoAllocScratchBytes : 0, stream);
}

int infv2_decode_compress_append(const void* k_pages, const int32_t* block_table, const int32_t* old_lens,
                                 const int32_t* new_lens, void* k_cmp, int B, int H_kv, int D, int block_size,
                                 int max_blocks, int num_pages, int max_new_blocks, void* stream) {
  int st = check_decode(B, H_kv, H_kv, D, block_size, max_blocks);
  if (st != INFV2_OK) return st;
  if (num_pages < 1 || max_new_blocks < 0 || max_new_blocks > max_blocks) return INFV2_ERR_INVALID;
  if (B == 0 || max_new_blocks == 0) return INFV2_OK;
  if (!tensor_ok(k_pages) || !tensor_ok(k_cmp) || !ints_ok(block_table) || !ints_ok(old_lens) ||
      !ints_ok(new_lens))
    return INFV2_ERR_INVALID;
  const AttnShape s = decode_shape(B, H_kv, H_kv, max_blocks, 0, 0, 1, 1.f, new_lens, block_table, num_pages);
  return hip_status(infv2::launch_compress_append(static_cast<const uint16_t*>(k_pages), s, old_lens,
                                                  static_cast<uint16_t*>(k_cmp), max_new_blocks,
                                                  static_cast<hipStream_t>(stream)));
}

int infv2_decode_select(const void* q, const void* k_cmp, const int32_t* seqlens, int32_t* blk_idx,
                        float* blk_score, int B, int H_q, int H_kv, int D, int block_size, int max_blocks,
                        int topk, int n_init, int n_local, float softmax_scale, void* stream) {
  int st = check_decode(B, H_q, H_kv, D, block_size, max_blocks);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (max_blocks > kMaxDecodeSelectBlocks) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || topk == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k_cmp) || !tensor_ok(blk_idx) || !ints_ok(seqlens)) return INFV2_ERR_INVALID;
  if (blk_score && !aligned(blk_score, 16)) return INFV2_ERR_INVALID;
  const AttnShape s = decode_shape(B, H_q, H_kv, max_blocks, topk, n_init, n_local, scale_log2(softmax_scale, D),
                                   seqlens, nullptr, 0);
  return hip_status(infv2::launch_select_blocks(static_cast<const uint16_t*>(q),
                                                static_cast<const uint16_t*>(k_cmp), blk_idx, blk_score, s,
                                                static_cast<hipStream_t>(stream)));
}

size_t infv2_decode_attn_workspace_bytes(int B, int H_q, int H_kv, int D, int block_size, int max_blocks,
                                         int topk) {
  if (check_decode(B, H_q, H_kv, D, block_size, max_blocks) != INFV2_OK || topk < 0) return 0;
  const AttnShape s = decode_shape(B, H_q, H_kv, max_blocks, topk, 0, 1, 1.f, nullptr, nullptr, 0);
  return round_up(infv2::attn_workspace_bytes(s), 256);
}

int infv2_decode_attn(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* seqlens, const int32_t* blk_idx, void* out, float* lse, int B, int H_q,
                      int H_kv, int D, int block_size, int max_blocks, int num_pages, int topk, int n_init,
                      int n_local, float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_decode(B, H_q, H_kv, D, block_size, max_blocks);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (max_blocks > kMaxSparseBlocks) return INFV2_ERR_UNSUPPORTED;
  if (num_pages < 1) return INFV2_ERR_INVALID;
  if (B == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k_pages) || !tensor_ok(v_pages) || !tensor_ok(out) || !ints_ok(block_table) ||
      !ints_ok(seqlens))
    return INFV2_ERR_INVALID;
  if (topk > 0 && !tensor_ok(blk_idx)) return INFV2_ERR_INVALID;
  if (lse && !aligned(lse, 16)) return INFV2_ERR_INVALID;
  const size_t need = infv2_decode_attn_workspace_bytes(B, H_q, H_kv, D, block_size, max_blocks, topk);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return INFV2_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return INFV2_ERR_INVALID;
  const AttnShape s = decode_shape(B, H_q, H_kv, max_blocks, topk, n_init, n_local, scale_log2(softmax_scale, D),
                                   seqlens, block_table, num_pages);
  return hip_status(infv2::launch_sparse_attn(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pages), static_cast<const uint16_t*>(v_pages),
      blk_idx, static_cast<uint16_t*>(out), lse, s, workspace, static_cast<hipStream_t>(stream)));
}

int infv2_decode_select_attn(const void* q, const void* k_cmp, const void* k_pages, const void* v_pages,
                             const int32_t* block_table, const int32_t* seqlens, int32_t* blk_idx, float* blk_score,
                             void* out, float* lse, int B, int H_q, int H_kv, int D, int block_size, int max_blocks,
                             int num_pages, int topk, int n_init, int n_local, float softmax_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int st = check_decode(B, H_q, H_kv, D, block_size, max_blocks);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (max_blocks > kMaxDecodeSelectBlocks) return INFV2_ERR_UNSUPPORTED;
  if (num_pages < 1) return INFV2_ERR_INVALID;
  if (B == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k_cmp) || !tensor_ok(k_pages) || !tensor_ok(v_pages) || !tensor_ok(out) ||
      !ints_ok(block_table) || !ints_ok(seqlens))
    return INFV2_ERR_INVALID;
  if (topk > 0 && !tensor_ok(blk_idx)) return INFV2_ERR_INVALID;
  if ((blk_score && !aligned(blk_score, 16)) || (lse && !aligned(lse, 16))) return INFV2_ERR_INVALID;
  const size_t need = infv2_decode_attn_workspace_bytes(B, H_q, H_kv, D, block_size, max_blocks, topk);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return INFV2_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return INFV2_ERR_INVALID;
  const AttnShape s = decode_shape(B, H_q, H_kv, max_blocks, topk, n_init, n_local, scale_log2(softmax_scale, D),
                                   seqlens, block_table, num_pages);
  return hip_status(infv2::launch_decode_select_attn(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cmp), static_cast<const uint16_t*>(k_pages),
      static_cast<const uint16_t*>(v_pages), blk_idx, blk_score, static_cast<uint16_t*>(out), lse, s, workspace,
      static_cast<hipStream_t>(stream)));
}

int infv2_compress_v(const void* v, void* v_cmp, int B, int H_kv, int S_k, int D, int block_size, void* stream) {
  // the values are compressed exactly like the keys
  return infv2_compress_k(v, v_cmp, B, H_kv, S_k, D, block_size, stream);
}

int infv2_compressed_attn_fwd(const void* q, const void* k_cmp, const void* v_cmp, const void* o_sparse, void* out,
                              float* lse, int B, int H_q, int H_kv, int S_q, int S_k, int D, int block_size,
                              float softmax_scale, float w_sparse, float w_cmp, void* stream) {
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  if (block_size < 1 || !isfinite(w_sparse) || !isfinite(w_cmp)) return INFV2_ERR_INVALID;
  if (block_size != infv2::kBS) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_q == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k_cmp) || !tensor_ok(v_cmp) || !tensor_ok(out)) return INFV2_ERR_INVALID;
  if ((o_sparse && !aligned(o_sparse, 16)) || (lse && !aligned(lse, 16))) return INFV2_ERR_INVALID;
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, 0, 0, 1, scale_log2(softmax_scale, D), 1);
  return hip_status(infv2::launch_compressed_attn(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cmp), static_cast<const uint16_t*>(v_cmp),
      static_cast<const uint16_t*>(o_sparse), static_cast<uint16_t*>(out), lse, s, w_sparse, w_cmp,
      static_cast<hipStream_t>(stream)));
}

int infv2_mixed_attn_fwd(const void* q, const void* k, const void* v, const int32_t* blk_idx, const void* k_cmp,
                         const void* v_cmp, void* out, float* lse, int B, int H_q, int H_kv, int S_q, int S_k, int D,
                         int block_size, int topk, int n_init, int n_local, float softmax_scale, float w_sparse,
                         float w_cmp, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(B, H_q, H_kv, S_q, S_k, D);
  if (st != INFV2_OK) return st;
  st = check_sparse_params(block_size, topk, n_init, n_local);
  if (st != INFV2_OK) return st;
  if (!isfinite(w_sparse) || !isfinite(w_cmp)) return INFV2_ERR_INVALID;
  if (num_blocks(S_k, block_size) > kMaxSparseBlocks) return INFV2_ERR_UNSUPPORTED;
  if (B == 0 || S_q == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(k_cmp) || !tensor_ok(v_cmp) || !tensor_ok(out))
    return INFV2_ERR_INVALID;
  if (topk > 0 && !tensor_ok(blk_idx)) return INFV2_ERR_INVALID;
  if (lse && !aligned(lse, 16)) return INFV2_ERR_INVALID;
  const size_t need = sparse_ws(B, H_q, H_kv, S_q, S_k, block_size, topk);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return INFV2_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return INFV2_ERR_INVALID;
  const AttnShape s = make_shape(B, H_q, H_kv, S_q, S_k, block_size, topk, n_init, n_local,
                                 scale_log2(softmax_scale, D), 1);
  return hip_status(infv2::launch_mixed_attn(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), blk_idx,
      static_cast<const uint16_t*>(k_cmp), static_cast<const uint16_t*>(v_cmp), static_cast<uint16_t*>(out), lse, s,
      w_sparse, w_cmp, workspace, static_cast<hipStream_t>(stream)));
}

int infv2_decode_compressed_attn(const void* q, const void* k_cmp, const void* v_cmp, const int32_t* seqlens,
                                 const void* o_sparse, void* out, float* lse, int B, int H_q, int H_kv, int D,
                                 int block_size, int max_blocks, float softmax_scale, float w_sparse, float w_cmp,
                                 void* stream) {
  int st = check_decode(B, H_q, H_kv, D, block_size, max_blocks);
  if (st != INFV2_OK) return st;
  if (!isfinite(w_sparse) || !isfinite(w_cmp)) return INFV2_ERR_INVALID;
  if (B == 0) return INFV2_OK;
  if (!tensor_ok(q) || !tensor_ok(k_cmp) || !tensor_ok(v_cmp) || !tensor_ok(out) || !ints_ok(seqlens))
    return INFV2_ERR_INVALID;
  if ((o_sparse && !aligned(o_sparse, 16)) || (lse && !aligned(lse, 16))) return INFV2_ERR_INVALID;
  const AttnShape s = decode_shape(B, H_q, H_kv, max_blocks, 0, 0, 1, scale_log2(softmax_scale, D), seqlens,
                                   nullptr, 0);
  return hip_status(infv2::launch_compressed_attn(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cmp), static_cast<const uint16_t*>(v_cmp),
      static_cast<const uint16_t*>(o_sparse), static_cast<uint16_t*>(out), lse, s, w_sparse, w_cmp,
      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
