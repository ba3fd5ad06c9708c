"""InfLLM-V2 block-sparse attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libinfv2.so`` (include/infv2.h).
Every function only checks and marshals arguments: all work runs in the HIP
kernels, enqueued on torch's current stream.  There is no CPU fallback: the
functions raise if the library has not been built or the tensors are not on
the GPU.

Names follow the C entry points without their ``infv2_`` prefix:
``compress_k``, ``select_blocks``, ``sparse_attn_fwd``, ``dense_attn_fwd``,
``attn_fwd``, the decode calls (``decode_*``), ``compress_v``,
``compressed_attn_fwd`` and ``mixed_attn_fwd``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinfv2.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
PATH_SPARSE, PATH_DENSE = 0, 1

_c_int, _c_size, _c_float, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

# name -> (restype, argtypes), mirroring include/infv2.h
SIGNATURES = {
    "infv2_status_string": (ctypes.c_char_p, [_c_int]),
    "infv2_abi_version": (_c_int, []),
    "infv2_compress_k": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "infv2_select_blocks": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 10 + [_c_float, _vp]),
    "infv2_select_blocks_strided_lse": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 10 + [_c_float, _c_int, _vp]),
    "infv2_sparse_workspace_bytes": (_c_size, [_c_int] * 8),
    "infv2_sparse_attn_fwd": (_c_int, [_vp] * 6 + [_c_int] * 10 + [_c_float, _vp, _c_size, _vp]),
    "infv2_sparse_bwd_workspace_bytes": (_c_size, [_c_int] * 8),
    "infv2_sparse_attn_bwd": (_c_int, [_vp] * 10 + [_c_int] * 10 + [_c_float, _vp, _c_size, _vp]),
    "infv2_dense_workspace_bytes": (_c_size, [_c_int] * 6),
    "infv2_dense_attn_fwd": (_c_int, [_vp] * 5 + [_c_int] * 6 + [_c_float, _c_int, _vp, _c_size, _vp]),
    "infv2_attn_workspace_bytes": (_c_size, [_c_int] * 9),
    "infv2_attn_path": (_c_int, [_c_int, _c_int]),
    "infv2_attn_fwd": (_c_int, [_vp] * 6 + [_c_int] * 10 + [_c_float, _c_int, _vp, _c_size, _vp]),
    "infv2_attn_fwd_noalloc": (_c_int, [_vp] * 6 + [_c_int] * 10 + [_c_float, _c_int, _vp]),
    "infv2_decode_compress_append": (_c_int, [_vp] * 5 + [_c_int] * 7 + [_vp]),
    "infv2_decode_select": (_c_int, [_vp] * 5 + [_c_int] * 9 + [_c_float, _vp]),
    "infv2_decode_attn_workspace_bytes": (_c_size, [_c_int] * 7),
    "infv2_decode_attn": (_c_int, [_vp] * 8 + [_c_int] * 10 + [_c_float, _vp, _c_size, _vp]),
    "infv2_decode_select_attn": (_c_int, [_vp] * 10 + [_c_int] * 10 + [_c_float, _vp, _c_size, _vp]),
    "infv2_compress_v": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "infv2_compressed_attn_fwd": (_c_int, [_vp] * 6 + [_c_int] * 7 + [_c_float] * 3 + [_vp]),
    "infv2_decode_compressed_attn": (_c_int, [_vp] * 7 + [_c_int] * 6 + [_c_float] * 3 + [_vp]),
    "infv2_mixed_attn_fwd": (_c_int, [_vp] * 8 + [_c_int] * 10 + [_c_float] * 3 + [_vp, _c_size, _vp]),
}

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libinfv2.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m trainable_block_sparse_mean_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class Infv2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load_library().infv2_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def _call(name: str, *args):
    st = getattr(load_library(), name)(*args)
    if st != OK:
        raise Infv2Error(name, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _scale(softmax_scale):
    return 0.0 if softmax_scale is None else float(softmax_scale)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def compress_k(k: torch.Tensor, block_size: int = 64) -> torch.Tensor:
    """Per-block key means, bf16 [B, H_kv, ceil(S_k/block_size), D]."""
    _need(k, "k", torch.bfloat16, 4)
    B, H_kv, S_k, D = k.shape
    nb = (S_k + block_size - 1) // block_size
    k_cmp = torch.empty(B, H_kv, nb, D, dtype=torch.bfloat16, device=k.device)
    _call("infv2_compress_k", _ptr(k), _ptr(k_cmp), B, H_kv, S_k, D, block_size, _stream())
    return k_cmp


def select_blocks(q: torch.Tensor, k_cmp: torch.Tensor, S_k: int, topk: int, n_init: int = 1,
                  n_local: int = 2, softmax_scale=None, block_size: int = 64, return_scores: bool = False):
    """Top-k blocks per (batch, KV group, query row): int32 [B, H_kv, S_q, topk],
    ascending, -1 padded; optionally also the group scores of those blocks."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cmp, "k_cmp", torch.bfloat16, 4)
    B, H_q, S_q, D = q.shape
    H_kv = k_cmp.shape[1]
    idx = torch.empty(B, H_kv, S_q, topk, dtype=torch.int32, device=q.device)
    score = torch.empty_like(idx, dtype=torch.float32) if return_scores else None
    _call("infv2_select_blocks", _ptr(q), _ptr(k_cmp), _ptr(idx), _ptr(score), B, H_q, H_kv, S_q, S_k, D,
          block_size, topk, n_init, n_local, _scale(softmax_scale), _stream())
    return (idx, score) if return_scores else idx


def select_blocks_strided_lse(q: torch.Tensor, k_cmp: torch.Tensor, S_k: int, topk: int, lse_stride: int,
                              n_init: int = 1, n_local: int = 2, softmax_scale=None, block_size: int = 64,
                              return_scores: bool = False):
    """select_blocks with the approximate per-head log-sum-exp over every
    lse_stride-th compressed block (1, 2, 4 or 8; 1 is exact)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cmp, "k_cmp", torch.bfloat16, 4)
    B, H_q, S_q, D = q.shape
    H_kv = k_cmp.shape[1]
    idx = torch.empty(B, H_kv, S_q, topk, dtype=torch.int32, device=q.device)
    score = torch.empty_like(idx, dtype=torch.float32) if return_scores else None
    _call("infv2_select_blocks_strided_lse", _ptr(q), _ptr(k_cmp), _ptr(idx), _ptr(score), B, H_q, H_kv, S_q, S_k,
          D, block_size, topk, n_init, n_local, _scale(softmax_scale), lse_stride, _stream())
    return (idx, score) if return_scores else idx


def sparse_attn_fwd(q, k, v, blk_idx, n_init: int = 1, n_local: int = 2, softmax_scale=None,
                    block_size: int = 64, return_lse: bool = True):
    """Attention over the initial, sliding-window and selected blocks.
    Returns (out bf16 [B,H_q,S_q,D], lse fp32 [B,H_q,S_q] or None)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    _need(blk_idx, "blk_idx", torch.int32, 4)
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    topk = blk_idx.shape[3]
    out = torch.empty_like(q)
    lse = torch.empty(B, H_q, S_q, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = load_library().infv2_sparse_workspace_bytes(B, H_q, H_kv, S_q, S_k, D, block_size, topk)
    ws = _workspace(nbytes, q.device)
    _call("infv2_sparse_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(blk_idx), _ptr(out), _ptr(lse),
          B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init, n_local, _scale(softmax_scale),
          _ptr(ws), ws.numel(), _stream())
    return out, lse


def sparse_attn_bwd(q, k, v, out, lse, dout, blk_idx, n_init: int = 1, n_local: int = 2, softmax_scale=None,
                    block_size: int = 64):
    """Gradients of sparse_attn_fwd with respect to q, k, v, given the forward's
    output and log-sum-exp and the gradient of the output.
    Returns (dq bf16 [B,H_q,S_q,D], dk, dv bf16 [B,H_kv,S_k,D])."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(blk_idx, "blk_idx", torch.int32, 4)
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    topk = blk_idx.shape[3]
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    nbytes = load_library().infv2_sparse_bwd_workspace_bytes(B, H_q, H_kv, S_q, S_k, D, block_size, topk)
    ws = _workspace(nbytes, q.device)
    _call("infv2_sparse_attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(blk_idx),
          _ptr(dq), _ptr(dk), _ptr(dv), B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init, n_local,
          _scale(softmax_scale), _ptr(ws), ws.numel(), _stream())
    return dq, dk, dv


def dense_attn_fwd(q, k, v, causal: bool = True, softmax_scale=None, return_lse: bool = True):
    """Dense (causal) GQA attention.  Returns (out, lse or None)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty(B, H_q, S_q, dtype=torch.float32, device=q.device) if return_lse else None
    ws = _workspace(load_library().infv2_dense_workspace_bytes(B, H_q, H_kv, S_q, S_k, D), q.device)
    _call("infv2_dense_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H_q, H_kv, S_q, S_k, D,
          _scale(softmax_scale), int(bool(causal)), _ptr(ws), ws.numel(), _stream())
    return out, lse


def decode_compress_append(k_pages, block_table, old_lens, new_lens, k_cmp, max_new_blocks: int,
                           block_size: int = 64):
    """Fill k_cmp (bf16 [B,H_kv,max_blocks,D], in place) with the compressed keys
    of the blocks of a paged cache that became complete when sequence b grew
    from old_lens[b] to new_lens[b] keys (at most max_new_blocks per sequence).
    k_pages bf16 [num_pages,H_kv,block_size,D]; block_table int32
    [B,max_blocks]; old_lens, new_lens int32 [B]."""
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(k_cmp, "k_cmp", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    for t, n in ((old_lens, "old_lens"), (new_lens, "new_lens")):
        _need(t, n, torch.int32, 1)
    num_pages, H_kv, _, D = k_pages.shape
    B, max_blocks = block_table.shape
    _call("infv2_decode_compress_append", _ptr(k_pages), _ptr(block_table), _ptr(old_lens), _ptr(new_lens),
          _ptr(k_cmp), B, H_kv, D, block_size, max_blocks, num_pages, max_new_blocks, _stream())
    return k_cmp


def decode_select(q, k_cmp, seqlens, topk: int, n_init: int = 1, n_local: int = 2, softmax_scale=None,
                  block_size: int = 64, return_scores: bool = False):
    """Block selection for one query per sequence (the last of its seqlens[b]
    keys).  q bf16 [B,H_q,D]; k_cmp bf16 [B,H_kv,max_blocks,D]; seqlens int32
    [B].  Returns blk_idx int32 [B,H_kv,topk] (and the group scores)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cmp, "k_cmp", torch.bfloat16, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, H_q, D = q.shape
    H_kv, max_blocks = k_cmp.shape[1], k_cmp.shape[2]
    idx = torch.empty(B, H_kv, topk, dtype=torch.int32, device=q.device)
    score = torch.empty(B, H_kv, topk, dtype=torch.float32, device=q.device) if return_scores else None
    _call("infv2_decode_select", _ptr(q), _ptr(k_cmp), _ptr(seqlens), _ptr(idx), _ptr(score), B, H_q, H_kv, D,
          block_size, max_blocks, topk, n_init, n_local, _scale(softmax_scale), _stream())
    return (idx, score) if return_scores else idx


def decode_attn(q, k_pages, v_pages, block_table, seqlens, blk_idx, n_init: int = 1, n_local: int = 2,
                softmax_scale=None, block_size: int = 64, return_lse: bool = True):
    """Block-sparse attention of one query per sequence over its paged keys.
    q bf16 [B,H_q,D]; k_pages, v_pages bf16 [num_pages,H_kv,block_size,D];
    block_table int32 [B,max_blocks]; seqlens int32 [B]; blk_idx int32
    [B,H_kv,topk].  Returns (out bf16 [B,H_q,D], lse fp32 [B,H_q] or None)."""
    _need(q, "q", torch.bfloat16, 3)
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n, torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seqlens, "seqlens", torch.int32, 1)
    _need(blk_idx, "blk_idx", torch.int32, 3)
    B, H_q, D = q.shape
    num_pages, H_kv = k_pages.shape[0], k_pages.shape[1]
    max_blocks = block_table.shape[1]
    topk = blk_idx.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = load_library().infv2_decode_attn_workspace_bytes(B, H_q, H_kv, D, block_size, max_blocks, topk)
    ws = _workspace(nbytes, q.device)
    _call("infv2_decode_attn", _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seqlens),
          _ptr(blk_idx), _ptr(out), _ptr(lse), B, H_q, H_kv, D, block_size, max_blocks, num_pages, topk, n_init,
          n_local, _scale(softmax_scale), _ptr(ws), ws.numel(), _stream())
    return out, lse


def decode_select_attn(q, k_cmp, k_pages, v_pages, block_table, seqlens, topk: int, n_init: int = 1,
                       n_local: int = 2, softmax_scale=None, block_size: int = 64, return_scores: bool = False):
    """decode_select then decode_attn in one launch (the same results).
    Returns (out bf16 [B,H_q,D], lse fp32 [B,H_q], blk_idx int32 [B,H_kv,topk]
    [, blk_score fp32 [B,H_kv,topk]])."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cmp, "k_cmp", torch.bfloat16, 4)
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n, torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, H_q, D = q.shape
    num_pages, H_kv = k_pages.shape[0], k_pages.shape[1]
    max_blocks = block_table.shape[1]
    if k_cmp.shape[2] != max_blocks:
        raise ValueError("k_cmp and block_table must hold the same number of blocks per sequence")
    idx = torch.empty(B, H_kv, topk, dtype=torch.int32, device=q.device)
    score = torch.empty(B, H_kv, topk, dtype=torch.float32, device=q.device) if return_scores else None
    out = torch.empty_like(q)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=q.device)
    nbytes = load_library().infv2_decode_attn_workspace_bytes(B, H_q, H_kv, D, block_size, max_blocks, topk)
    ws = _workspace(nbytes, q.device)
    _call("infv2_decode_select_attn", _ptr(q), _ptr(k_cmp), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
          _ptr(seqlens), _ptr(idx), _ptr(score), _ptr(out), _ptr(lse), B, H_q, H_kv, D, block_size, max_blocks,
          num_pages, topk, n_init, n_local, _scale(softmax_scale), _ptr(ws), ws.numel(), _stream())
    return (out, lse, idx, score) if return_scores else (out, lse, idx)


def compress_v(v: torch.Tensor, block_size: int = 64) -> torch.Tensor:
    """Per-block value means, bf16 [B, H_kv, ceil(S_k/block_size), D]."""
    _need(v, "v", torch.bfloat16, 4)
    B, H_kv, S_k, D = v.shape
    nb = (S_k + block_size - 1) // block_size
    v_cmp = torch.empty(B, H_kv, nb, D, dtype=torch.bfloat16, device=v.device)
    _call("infv2_compress_v", _ptr(v), _ptr(v_cmp), B, H_kv, S_k, D, block_size, _stream())
    return v_cmp


def compressed_attn_fwd(q, k_cmp, v_cmp, S_k: int, o_sparse=None, w_sparse: float = 0.0, w_cmp: float = 1.0,
                        softmax_scale=None, block_size: int = 64, out=None, return_lse: bool = True):
    """Compressed-attention branch, causal over whole blocks, optionally mixed
    with another pattern's output: out = w_cmp * O_cmp (+ w_sparse * o_sparse).
    q bf16 [B,H_q,S_q,D]; k_cmp, v_cmp bf16 [B,H_kv,ceil(S_k/64),D].  ``out``
    may be given (also ``out is o_sparse``, in place).  Returns (out, lse)."""
    _need(q, "q", torch.bfloat16, 4)
    for t, n in ((k_cmp, "k_cmp"), (v_cmp, "v_cmp")):
        _need(t, n, torch.bfloat16, 4)
    if o_sparse is not None:
        _need(o_sparse, "o_sparse", torch.bfloat16, 4)
    B, H_q, S_q, D = q.shape
    H_kv = k_cmp.shape[1]
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.bfloat16, 4)
    lse = torch.empty(B, H_q, S_q, dtype=torch.float32, device=q.device) if return_lse else None
    _call("infv2_compressed_attn_fwd", _ptr(q), _ptr(k_cmp), _ptr(v_cmp), _ptr(o_sparse), _ptr(out), _ptr(lse),
          B, H_q, H_kv, S_q, S_k, D, block_size, _scale(softmax_scale), float(w_sparse), float(w_cmp), _stream())
    return out, lse


def mixed_attn_fwd(q, k, v, blk_idx, k_cmp, v_cmp, w_sparse: float, w_cmp: float, n_init: int = 1,
                   n_local: int = 2, softmax_scale=None, block_size: int = 64, return_lse: bool = True):
    """Block-sparse attention and the compressed branch in one call:
    out = w_sparse * O_sparse + w_cmp * O_cmp.  Arguments as sparse_attn_fwd
    plus k_cmp, v_cmp (bf16 [B,H_kv,ceil(S_k/64),D]).  Returns (out, lse of
    the sparse attention)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (k_cmp, "k_cmp"), (v_cmp, "v_cmp")):
        _need(t, n, torch.bfloat16, 4)
    _need(blk_idx, "blk_idx", torch.int32, 4)
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    topk = blk_idx.shape[3]
    out = torch.empty_like(q)
    lse = torch.empty(B, H_q, S_q, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = load_library().infv2_sparse_workspace_bytes(B, H_q, H_kv, S_q, S_k, D, block_size, topk)
    ws = _workspace(nbytes, q.device)
    _call("infv2_mixed_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(blk_idx), _ptr(k_cmp), _ptr(v_cmp), _ptr(out),
          _ptr(lse), B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init, n_local, _scale(softmax_scale),
          float(w_sparse), float(w_cmp), _ptr(ws), ws.numel(), _stream())
    return out, lse


def decode_compressed_attn(q, k_cmp, v_cmp, seqlens, o_sparse=None, w_sparse: float = 0.0, w_cmp: float = 1.0,
                           softmax_scale=None, block_size: int = 64, return_lse: bool = True):
    """Compressed-attention branch of one query per sequence.  q bf16
    [B,H_q,D]; k_cmp, v_cmp bf16 [B,H_kv,max_blocks,D]; seqlens int32 [B];
    o_sparse bf16 [B,H_q,D] or None.  Returns (out, lse)."""
    _need(q, "q", torch.bfloat16, 3)
    for t, n in ((k_cmp, "k_cmp"), (v_cmp, "v_cmp")):
        _need(t, n, torch.bfloat16, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    if o_sparse is not None:
        _need(o_sparse, "o_sparse", torch.bfloat16, 3)
    B, H_q, D = q.shape
    H_kv, max_blocks = k_cmp.shape[1], k_cmp.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=q.device) if return_lse else None
    _call("infv2_decode_compressed_attn", _ptr(q), _ptr(k_cmp), _ptr(v_cmp), _ptr(seqlens), _ptr(o_sparse),
          _ptr(out), _ptr(lse), B, H_q, H_kv, D, block_size, max_blocks, _scale(softmax_scale), float(w_sparse),
          float(w_cmp), _stream())
    return out, lse


class AttnPlan:
    """Pre-sized buffers for repeated ``attn_fwd`` calls on one shape."""

    def __init__(self, B, H_q, H_kv, S_q, S_k, D=128, block_size=64, topk=64, n_init=1, n_local=2,
                 switch_len=0, softmax_scale=None, device="cuda", with_lse=True, with_idx=False):
        self.args = (B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init, n_local)
        self.switch_len = switch_len
        self.scale = _scale(softmax_scale)
        self.dense = load_library().infv2_attn_path(S_k, switch_len) == PATH_DENSE
        nbytes = load_library().infv2_attn_workspace_bytes(B, H_q, H_kv, S_q, S_k, D, block_size, topk,
                                                           switch_len)
        self.ws = _workspace(nbytes, device)
        self.out = torch.empty(B, H_q, S_q, D, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(B, H_q, S_q, dtype=torch.float32, device=device) if with_lse else None
        self.idx = (torch.empty(B, H_kv, S_q, topk, dtype=torch.int32, device=device)
                    if with_idx and not self.dense else None)

    def run(self, q, k, v):
        B, H_q, H_kv, S_q, S_k, D, bs, topk, n_init, n_local = self.args
        _call("infv2_attn_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(self.out), _ptr(self.lse), _ptr(self.idx),
              B, H_q, H_kv, S_q, S_k, D, bs, topk, n_init, n_local, self.scale, self.switch_len,
              _ptr(self.ws), self.ws.numel(), _stream())
        return self.out, self.lse


def attn_fwd(q, k, v, block_size: int = 64, topk: int = 64, n_init: int = 1, n_local: int = 2,
             switch_len: int = 0, softmax_scale=None, return_idx: bool = False):
    """The dense/sparse switch: dense causal attention if S_k <= switch_len,
    else compress -> select -> sparse.  Returns dict(out, lse, path, blk_idx)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    plan = AttnPlan(B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init, n_local, switch_len, softmax_scale,
                    q.device, True, return_idx)
    out, lse = plan.run(q, k, v)
    return dict(out=out, lse=lse, path="dense" if plan.dense else "sparse", blk_idx=plan.idx)


def attn_fwd_noalloc(q, k, v, out, lse, blk_idx=None, block_size: int = 64, topk: int = 64, n_init: int = 1,
                     n_local: int = 2, switch_len: int = 0, softmax_scale=None) -> None:
    """infv2_attn_fwd_noalloc: the switch into caller-given out (bf16, shaped
    like q), lse (fp32 [B,H_q,S_q] or None) and optional blk_idx, with the
    library's fixed per-GPU scratch as its workspace (nothing is allocated)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, torch.bfloat16, 4)
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    _call("infv2_attn_fwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(blk_idx),
          B, H_q, H_kv, S_q, S_k, D, block_size, topk, n_init, n_local, _scale(softmax_scale), switch_len,
          _stream())


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
