"""fp64 CPU oracle for InfLLM-V2 dense-sparse switchable attention (forward and
the block-sparse attention backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

Plain NumPy, float64 throughout.  Every function follows one passage of the
pages, named in its docstring as  [page title, section].  The pages are:

  * "Infllm V2 Dense Sparse Switchable Attention" (skill page), with the
    sections Architecture Overview; Step 1: Dense Attention Layer Foundation;
    Step 2: Sparse Pattern Selection Module; Step 3: Switchable Attention with
    Pattern Router; Step 5: Training and Fine-tuning Procedure; Practical
    Guidance (When NOT to Use, Common Pitfalls).
  * "InfLLM-V2: Dense-Sparse Switchable Attention for Seamless Short-to-Long
    Adaptation" (paper page), Abstract.
  * The InfLLM-V2 news summary (reportify), sections Model Advantages,
    Technical Mechanism and Performance Evaluation.

Readings where the pages are silent or contradict one another are stated in
each docstring (they are listed together in the design notes of the repo).

Conventions
-----------
* Tensors are [B, H, S, D] (skill page, Step 2, shape docstrings).  bf16
  inputs arrive as uint16 bit patterns and are widened exactly to float64.
* Query head h uses KV head h // G, G = H_q / H_kv (consecutive GQA groups).
* Query row r sits at absolute position i = (S_k - S_q) + r (bottom-right
  alignment, so one decode query is the last token of the cache).
* Block j holds key positions [j*BS, (j+1)*BS).
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# bf16 <-> float64
# ---------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 directly to bf16 (8 significant bits), nearest-even.

    Returns uint16 bit patterns.  The rounding is done in float64 on the
    integer significand (np.round rounds halves to even), so there is no
    intermediate float32 rounding step.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2**-126 bf16 is subnormal
    quantum = np.ldexp(1.0, e - 8)          # weight of the last kept bit
    r = np.round(x / quantum) * quantum     # exact: quantum is a power of two
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)          # exact (<= 8 significant bits) or inf
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# a1: key compression
# ---------------------------------------------------------------------------


def compress_k(k: np.ndarray, block_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Block-mean compression of the keys.

    [skill page, Step 2: Sparse Pattern Selection Module, compressed_attention]:
    pad the sequence with zeros to a multiple of the block size, view it as
    non-overlapping blocks and take the mean over each block's tokens.  The
    divisor is the block size also for the zero-padded last block.

    Reading: only K is compressed on the hot path (the compressed keys feed
    block selection); the mean is rounded once to bf16, nearest-even.

    k: float64 [B, H, S, D].  Returns (k_cmp_bits uint16, k_cmp float64), both
    [B, H, ceil(S/BS), D]; k_cmp holds the bf16 values widened back.
    """
    B, H, S, D = k.shape
    nb = (S + block_size - 1) // block_size
    padded = np.zeros((B, H, nb * block_size, D), dtype=np.float64)
    padded[:, :, :S, :] = k
    mean = padded.reshape(B, H, nb, block_size, D).mean(axis=3)
    bits = f64_to_bf16(mean)
    return bits, bf16_to_f64(bits)


# ---------------------------------------------------------------------------
# a2: group-summed block scores
# ---------------------------------------------------------------------------


def visible_blocks(i: int, block_size: int) -> int:
    """Number of compressed blocks fully at or before position i: floor((i+1)/BS).

    Reading: a compressed key stands for its whole block, so a query may only
    score blocks whose every token is visible to it; the pages require the
    sparse patterns to stay causal [skill page, Practical Guidance, When NOT
    to Use].  The unmasked softmax of compressed_attention is not followed.
    """
    return (i + 1) // block_size


def group_scores(q: np.ndarray, k_cmp: np.ndarray, b: int, g: int, i: int,
                 r: int, G: int, scale: float, block_size: int) -> np.ndarray:
    """Group score sigma_j of every fully visible block j for one query row.

    [skill page, Architecture Overview, Hardware Kernel] sums normalised scores
    over the heads of a head group, the normalisation being a log-sum-exp;
    [skill page, Step 2, compressed_attention] gives the scores themselves:
    softmax over the scaled products of the query with the compressed keys.

    For each head h of group g:  z_hj = scale * <q_h, k_cmp_j>,
    p_hj = exp(z_hj - logsumexp_j z_hj); then sigma_j = sum_h p_hj.
    The log-sum-exp is exact (the pages leave its approximation undefined).

    Returns float64 [nv]; empty when no block is fully visible.
    """
    nv = visible_blocks(i, block_size)
    if nv == 0:
        return np.zeros(0)
    qh = q[b, g * G:(g + 1) * G, r, :]                 # [G, D]
    z = scale * (qh @ k_cmp[b, g, :nv, :].T)            # [G, nv]
    zmax = z.max(axis=1, keepdims=True)
    lse = zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True))
    p = np.exp(z - lse)
    return p.sum(axis=0)


def group_scores_strided_lse(q: np.ndarray, k_cmp: np.ndarray, b: int, g: int, i: int, r: int, G: int,
                             scale: float, block_size: int, stride: int) -> np.ndarray:
    """group_scores with an approximate per-head log-sum-exp.

    [skill page, Architecture Overview, Hardware Kernel] names an LSE
    approximation in its first pass without defining it.  Reading: the
    normaliser of head h is estimated from every stride-th visible compressed
    block, block R*x (R = stride) standing for the R blocks R*x .. R*x+R-1,
    the last group for its visible count w_x = min(R, nv - R*x):
        LSE_h ~ log sum_x w_x exp(z_h,R*x).
    The scores themselves (pass 2) are exact; stride 1 is group_scores.
    """
    nv = visible_blocks(i, block_size)
    if nv == 0:
        return np.zeros(0)
    qh = q[b, g * G:(g + 1) * G, r, :]                  # [G, D]
    z = scale * (qh @ k_cmp[b, g, :nv, :].T)            # [G, nv]
    xs = np.arange(0, nv, stride)                       # sampled blocks R*x
    w = np.minimum(stride, nv - xs).astype(np.float64)  # blocks each one stands for
    zs = z[:, xs] + np.log(w)[None, :]
    zmax = zs.max(axis=1, keepdims=True)
    lse = zmax + np.log(np.exp(zs - zmax).sum(axis=1, keepdims=True))
    return np.exp(z - lse).sum(axis=0)


def select_blocks_strided_lse(q: np.ndarray, k_cmp: np.ndarray, S_k: int, topk: int, n_init: int, n_local: int,
                              block_size: int, scale: float, stride: int, rows=None, return_scores: bool = False):
    """select_blocks with the approximate normaliser of group_scores_strided_lse."""
    B, H_q, S_q, _ = q.shape
    H_kv = k_cmp.shape[1]
    G = H_q // H_kv
    off = S_k - S_q
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    idx = np.full((B, H_kv, rows.size, topk), -1, dtype=np.int32)
    scores = {}
    for b in range(B):
        for g in range(H_kv):
            for n, r in enumerate(rows):
                i = off + int(r)
                sig = group_scores_strided_lse(q, k_cmp, b, g, i, int(r), G, scale, block_size, stride)
                idx[b, g, n] = select_row(sig, i, block_size, topk, n_init, n_local)
                if return_scores:
                    scores[(b, g, int(r))] = sig
    return (idx, scores) if return_scores else idx


# ---------------------------------------------------------------------------
# a3: top-k block selection
# ---------------------------------------------------------------------------


def candidates(i: int, block_size: int, n_init: int, n_local: int) -> np.ndarray:
    """Candidate blocks of the query at position i: n_init <= j <= qb - n_local.

    The initial blocks and the sliding-window blocks are always attended
    (see forced_blocks), so they are not candidates; every candidate is fully
    visible because n_local >= 1.
    """
    qb = i // block_size
    lo, hi = n_init, qb - n_local
    if hi < lo:
        return np.zeros(0, dtype=np.int64)
    return np.arange(lo, hi + 1, dtype=np.int64)


def select_row(sigma: np.ndarray, i: int, block_size: int, topk: int,
               n_init: int, n_local: int) -> np.ndarray:
    """Top-k candidate blocks of one query row, ascending, -1 padded to topk.

    [skill page, Step 2, selected_attention] keeps the top-k per query
    position; [news summary, Technical Mechanism] makes the unit of selection
    a block.  Order: larger sigma first; equal sigma goes to the lower block
    index.  With fewer candidates than topk all of them are kept.
    """
    c = candidates(i, block_size, n_init, n_local)
    out = np.full(topk, -1, dtype=np.int32)
    if topk == 0 or c.size == 0:
        return out
    order = np.lexsort((c, -sigma[c]))           # primary -sigma, then index
    chosen = np.sort(c[order[:min(topk, c.size)]])
    out[:chosen.size] = chosen
    return out


def select_blocks(q: np.ndarray, k_cmp: np.ndarray, S_k: int, topk: int,
                  n_init: int, n_local: int, block_size: int, scale: float,
                  rows=None, return_scores: bool = False):
    """Selected block indices for every (b, KV group g, query row r).

    q float64 [B, H_q, S_q, D]; k_cmp float64 [B, H_kv, NB, D].
    Returns int32 [B, H_kv, len(rows), topk]; with return_scores also a list
    (same order) of the float64 sigma vectors per row.
    """
    B, H_q, S_q, _ = q.shape
    H_kv = k_cmp.shape[1]
    G = H_q // H_kv
    off = S_k - S_q
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    idx = np.full((B, H_kv, rows.size, topk), -1, dtype=np.int32)
    scores = {}
    for b in range(B):
        for g in range(H_kv):
            for n, r in enumerate(rows):
                i = off + int(r)
                sig = group_scores(q, k_cmp, b, g, i, int(r), G, scale, block_size)
                idx[b, g, n] = select_row(sig, i, block_size, topk, n_init, n_local)
                if return_scores:
                    scores[(b, g, int(r))] = sig
    return (idx, scores) if return_scores else idx


# ---------------------------------------------------------------------------
# a4: block-sparse attention
# ---------------------------------------------------------------------------


def forced_blocks(i: int, block_size: int, n_init: int, n_local: int) -> list[int]:
    """Blocks every query attends regardless of scores.

    Reading: the first n_init blocks (initial / sink blocks) and a causal,
    block-granular sliding window made of the query's own block and the
    n_local - 1 blocks before it.  [skill page, Step 2, sliding_attention]
    keeps local context; [skill page, Practical Guidance, When NOT to Use]
    requires the window to respect causality, so its symmetric token window
    is not followed.
    """
    qb = i // block_size
    f = set(range(0, min(n_init, qb + 1)))
    f.update(range(max(qb - n_local + 1, 0), qb + 1))
    return sorted(f)


def attend_keys(i: int, blocks, block_size: int, S_k: int) -> np.ndarray:
    """Key positions t <= i inside the given blocks (causal within a block)."""
    ts = [np.arange(j * block_size, min((j + 1) * block_size, S_k)) for j in sorted(set(blocks))]
    t = np.concatenate(ts) if ts else np.zeros(0, dtype=np.int64)
    return t[t <= i]


def _softmax_attend(qh: np.ndarray, kk: np.ndarray, vv: np.ndarray, scale: float):
    """softmax(scale * q k^T) v and its natural-log log-sum-exp, per head.

    [skill page, Step 1: Dense Attention Layer Foundation]: scores are the
    scaled query-key products, weights their softmax, the context the weighted
    sum of values.  qh [G, D], kk/vv [T, D].
    """
    z = scale * (qh @ kk.T)                                  # [G, T]
    zmax = z.max(axis=1, keepdims=True)
    w = np.exp(z - zmax)
    l = w.sum(axis=1, keepdims=True)
    return (w / l) @ vv, (zmax + np.log(l))[:, 0]


def sparse_attn(q, k, v, blk_idx, block_size: int, n_init: int, n_local: int,
                scale: float, rows=None):
    """Attention restricted to the forced blocks and the selected blocks.

    [news summary, Technical Mechanism]: attention is computed only on the
    selected subsets of key-value blocks.  Attended set of the query at
    position i: forced_blocks(i) union the row's selected blocks (entries
    >= 0 of blk_idx); keys beyond i are masked (causal).

    q [B,H_q,S_q,D]; k, v [B,H_kv,S_k,D]; blk_idx int [B,H_kv,n_rows,topk]
    aligned with ``rows``.  Returns (out [B,H_q,n_rows,D], lse [B,H_q,n_rows]).
    """
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    G = H_q // H_kv
    off = S_k - S_q
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    out = np.zeros((B, H_q, rows.size, D))
    lse = np.zeros((B, H_q, rows.size))
    for b in range(B):
        for g in range(H_kv):
            for n, r in enumerate(rows):
                i = off + int(r)
                sel = [int(j) for j in blk_idx[b, g, n] if j >= 0]
                t = attend_keys(i, forced_blocks(i, block_size, n_init, n_local) + sel,
                                block_size, S_k)
                o, m = _softmax_attend(q[b, g * G:(g + 1) * G, int(r), :],
                                       k[b, g, t, :], v[b, g, t, :], scale)
                out[b, g * G:(g + 1) * G, n, :] = o
                lse[b, g * G:(g + 1) * G, n] = m
    return out, lse


# ---------------------------------------------------------------------------
# decode over a paged, variable-length cache
# ---------------------------------------------------------------------------


def paged_sequence(pages: np.ndarray, table_row, length: int, block_size: int) -> np.ndarray:
    """The keys (or values) of one sequence of a paged cache, in order.

    A paged cache stores each sequence's key blocks in pages; logical block j
    of the sequence is page table_row[j], one block of every KV head.  The
    sequence is its blocks concatenated in table order and cut to its length.

    pages [num_pages, H, BS, D]; returns [H, length, D].
    """
    nb = (length + block_size - 1) // block_size
    blocks = [pages[int(table_row[j])] for j in range(nb)]
    return np.concatenate(blocks, axis=1)[:, :length, :]


def decode_paged(q, k_pages, v_pages, block_table, seqlens, block_size: int, topk: int,
                 n_init: int, n_local: int, scale: float):
    """One decode step over a paged, variable-length cache.

    [news summary, Performance Evaluation]: the method is applied at decode
    time too.  Each sequence b has seqlens[b] keys; its one new query sits at
    the last key position (bottom-right alignment).  Per sequence this is
    exactly compress_k -> select_blocks -> sparse_attn on the sequence's
    contiguous keys and values (paged_sequence), with S_q = 1.

    q [B, H_q, D]; k_pages, v_pages [num_pages, H_kv, BS, D]; block_table
    int [B, max_blocks]; seqlens int [B].  Returns (k_cmp per sequence: list
    of [H_kv, ceil(L/BS), D], blk_idx int32 [B, H_kv, topk], out [B, H_q, D],
    lse [B, H_q]).
    """
    B, H_q, D = q.shape
    H_kv = k_pages.shape[1]
    idx = np.full((B, H_kv, topk), -1, dtype=np.int32)
    out = np.zeros((B, H_q, D))
    lse = np.zeros((B, H_q))
    kcs = []
    for b in range(B):
        L = int(seqlens[b])
        kb = paged_sequence(k_pages, block_table[b], L, block_size)[None]
        vb = paged_sequence(v_pages, block_table[b], L, block_size)[None]
        qb = q[b][None, :, None, :]
        _, kc = compress_k(kb, block_size)
        kcs.append(kc[0])
        ib = select_blocks(qb, kc, L, topk, n_init, n_local, block_size, scale)
        idx[b] = ib[0, :, 0, :]
        ob, lb = sparse_attn(qb, kb, vb, ib, block_size, n_init, n_local, scale)
        out[b] = ob[0, :, 0, :]
        lse[b] = lb[0, :, 0]
    return kcs, idx, out, lse


# ---------------------------------------------------------------------------
# a5: dense attention and the switch
# ---------------------------------------------------------------------------


def dense_attn(q, k, v, scale: float, causal: bool = True, rows=None):
    """Full (causal) GQA attention.

    [skill page, Step 1: Dense Attention Layer Foundation]: softmax of the
    scaled products over all keys, then the weighted sum of values.  Causal
    here means key t is visible to the query at position i iff t <= i.
    Returns (out [B,H_q,n_rows,D], lse [B,H_q,n_rows]).
    """
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    G = H_q // H_kv
    off = S_k - S_q
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    out = np.zeros((B, H_q, rows.size, D))
    lse = np.zeros((B, H_q, rows.size))
    for b in range(B):
        for g in range(H_kv):
            for n, r in enumerate(rows):
                i = off + int(r)
                t = np.arange(i + 1) if causal else np.arange(S_k)
                o, m = _softmax_attend(q[b, g * G:(g + 1) * G, int(r), :],
                                       k[b, g, t, :], v[b, g, t, :], scale)
                out[b, g * G:(g + 1) * G, n, :] = o
                lse[b, g * G:(g + 1) * G, n] = m
    return out, lse


def uses_dense(S_k: int, switch_len: int) -> bool:
    """[skill page, Step 3: Switchable Attention with Pattern Router]: a
    sequence no longer than the threshold takes the dense path (<=)."""
    return S_k <= switch_len


def attention(q, k, v, block_size: int, topk: int, n_init: int, n_local: int,
              switch_len: int, scale: float | None = None, rows=None):
    """The switch: dense causal attention for S_k <= switch_len, otherwise
    compress -> select -> block-sparse attention.

    [paper page, Abstract]: dense attention for short inputs, sparse for long.
    [news summary, Technical Mechanism]: block selection, then attention on
    the selected subsets.  Returns dict(out, lse, path, blk_idx, k_cmp_bits).
    """
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    S_k = k.shape[2]
    if uses_dense(S_k, switch_len):
        o, l = dense_attn(q, k, v, scale, causal=True, rows=rows)
        return dict(out=o, lse=l, path="dense", blk_idx=None, k_cmp_bits=None)
    bits, kc = compress_k(k, block_size)
    idx = select_blocks(q, kc, S_k, topk, n_init, n_local, block_size, scale, rows=rows)
    o, l = sparse_attn(q, k, v, idx, block_size, n_init, n_local, scale, rows=rows)
    return dict(out=o, lse=l, path="sparse", blk_idx=idx, k_cmp_bits=bits)


# ---------------------------------------------------------------------------
# The compressed-attention branch and the mix of patterns (next row)
# ---------------------------------------------------------------------------


def compress_v(v: np.ndarray, block_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Block-mean compression of the values.

    [skill page, Step 2, compressed_attention]: the values are compressed
    exactly like the keys (zero padding, mean over each block's tokens, the
    divisor being the block size).  Rounded once to bf16, nearest-even.
    Returns (v_cmp_bits uint16, v_cmp float64), both [B, H, ceil(S/BS), D].
    """
    return compress_k(v, block_size)


def compressed_attn(q, k_cmp, v_cmp, S_k: int, block_size: int, scale: float, rows=None):
    """Output of the compressed-attention branch.

    [skill page, Step 2, compressed_attention]: every query attends the
    compressed keys with a softmax of the scaled products and takes the
    weighted sum of the compressed values.

    Readings: causal like block scoring (visible_blocks): the query at
    position i sees only the nv = floor((i+1)/BS) blocks that lie wholly at
    or before it; the sketch's unmasked softmax would let it read values of
    later tokens.  The sketch's last step (repeating each row once per token
    of a block) does not fit its own shapes, whose rows are already one per
    query; the output here is one row per query.  A query that sees no block
    (its position is below BS - 1) gets a zero output and a log-sum-exp of
    -inf.

    q [B,H_q,S_q,D]; k_cmp, v_cmp float64 [B,H_kv,NB,D] (NB >= the visible
    blocks of the last query).  Returns (out [B,H_q,n_rows,D], lse
    [B,H_q,n_rows]) for the query rows ``rows`` (default: all).
    """
    B, H_q, S_q, D = q.shape
    H_kv = k_cmp.shape[1]
    G = H_q // H_kv
    off = S_k - S_q
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    out = np.zeros((B, H_q, rows.size, D))
    lse = np.full((B, H_q, rows.size), -np.inf)
    for b in range(B):
        for g in range(H_kv):
            for n, r in enumerate(rows):
                nv = visible_blocks(off + int(r), block_size)
                if nv == 0:
                    continue
                o, m = _softmax_attend(q[b, g * G:(g + 1) * G, int(r), :],
                                       k_cmp[b, g, :nv, :], v_cmp[b, g, :nv, :], scale)
                out[b, g * G:(g + 1) * G, n, :] = o
                lse[b, g * G:(g + 1) * G, n] = m
    return out, lse


def mix_patterns(outputs, weights) -> np.ndarray:
    """Weighted sum of pattern outputs.

    [skill page, Step 3: Switchable Attention with Pattern Router]: the
    sparse context is the sum of the pattern outputs, each multiplied by its
    coefficient.  Readings: the coefficients are given numbers (the page
    learns them through a softmax over a trainable vector, which a
    parameter-free method has no place for); the block-sparse output, whose
    one softmax already spans the selected, initial and window blocks, is one
    pattern and the compressed branch another.
    """
    out = np.zeros(np.shape(outputs[0]))
    for w, o in zip(weights, outputs):
        out = out + float(w) * np.asarray(o, dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# Backward of the block-sparse attention (next row: training)
# ---------------------------------------------------------------------------


def _softmax_attend_grad(qh: np.ndarray, kk: np.ndarray, vv: np.ndarray, do: np.ndarray,
                         scale: float, magnitudes: bool = False):
    """Gradients of o = softmax(scale * q k^T) v for one token's head group.

    [skill page, Step 5: Training and Fine-tuning Procedure]: the attention
    is trained by back-propagating a loss through it; this is the chain rule
    through the forward of [skill page, Step 1].  With p the softmax weights,
    dp = dO v^T, and the softmax Jacobian dz = p * (dp - <dO, o>):
    dq = scale * dz k,  dk = scale * dz^T q,  dv = p^T dO.
    qh, do [G, D]; kk, vv [T, D].  Returns (dq [G, D], dk [T, D], dv [T, D]).
    With ``magnitudes`` it also returns the same sums taken over absolute
    values, with |dz| replaced by p * (|dp| + |<dO, o>|): the size of the
    terms a rounded computation adds up (a scale for its rounding error).
    """
    z = scale * (qh @ kk.T)                                   # [G, T]
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ vv                                                # [G, D]
    dp = do @ vv.T                                            # [G, T]
    d = (do * o).sum(axis=1, keepdims=True)
    dz = p * (dp - d)
    grads = (scale * (dz @ kk), scale * (dz.T @ qh), p.T @ do)
    if not magnitudes:
        return grads
    mz = p * (np.abs(dp) + np.abs(d))
    return grads + (scale * (mz @ np.abs(kk)), scale * (mz.T @ np.abs(qh)), p.T @ np.abs(do))


def sparse_attn_bwd(q, k, v, dout, blk_idx, block_size: int, n_init: int, n_local: int,
                    scale: float, magnitudes: bool = False):
    """Gradients of the block-sparse attention with respect to q, k and v.

    [skill page, Step 5: Training and Fine-tuning Procedure] applied to the
    attention of ``sparse_attn``: the attended key set of each query is the
    same (forced blocks, selected blocks, causal inside a block), and the
    selection itself is a discrete choice with no gradient, so gradients flow
    only through the attention over that set.  The key and value gradients
    of a KV head sum over every query token and every head of its group that
    attends the key.

    q, dout [B,H_q,S_q,D]; k, v [B,H_kv,S_k,D]; blk_idx int [B,H_kv,S_q,topk].
    Returns (dq [B,H_q,S_q,D], dk [B,H_kv,S_k,D], dv [B,H_kv,S_k,D]), and with
    ``magnitudes`` also the absolute-value sums of _softmax_attend_grad in
    the same shapes.
    """
    B, H_q, S_q, D = q.shape
    H_kv, S_k = k.shape[1], k.shape[2]
    G = H_q // H_kv
    off = S_k - S_q
    res = [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
    if magnitudes:
        res += [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
    for b in range(B):
        for g in range(H_kv):
            hs = slice(g * G, (g + 1) * G)
            for r in range(S_q):
                i = off + r
                sel = [int(j) for j in blk_idx[b, g, r] if j >= 0]
                t = attend_keys(i, forced_blocks(i, block_size, n_init, n_local) + sel, block_size, S_k)
                parts = _softmax_attend_grad(q[b, hs, r, :], k[b, g, t, :], v[b, g, t, :],
                                             dout[b, hs, r, :], scale, magnitudes)
                for n in range(0, len(res), 3):
                    res[n][b, hs, r, :] = parts[n]
                    res[n + 1][b, g, t, :] += parts[n + 1]
                    res[n + 2][b, g, t, :] += parts[n + 2]
    return tuple(res)

