"""Seeded random shapes through every prefill entry point vs the fp64 oracle.

Each case draws B, the KV heads, the group size G (powers of two and not),
S_k, S_q <= S_k, topk (0 included), n_init and n_local, then checks, stage by
stage as in test_gpu_parity: the key and value compression bit for bit, the
selection (near-tie rule), the block-sparse attention on the GPU's selection,
the compressed-attention branch on the GPU's compressed keys and values, and
the dense attention.  Long query ranges are checked on sampled rows (always
including the first and last 70).  Tolerances are in tests/parity.py.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.infv2_oracle as O
import trainable_block_sparse_mean_amd as tb
from tests.parity import assert_attn_close, check_selection, np64, sparse_rows_q

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BS = 64


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def draw_case(seed):
    r = np.random.default_rng(seed)
    H_kv = int(r.choice([1, 2, 3, 4]))
    G = int(r.choice([1, 2, 3, 4, 5, 7, 8, 16]))
    S_k = int(r.integers(1, 3200))
    S_q = int(r.choice([S_k, int(r.integers(1, S_k + 1))]))
    return dict(B=int(r.integers(1, 3)), H_kv=H_kv, G=G, S_k=S_k, S_q=S_q, topk=int(r.choice([0, 1, 5, 16, 40])),
                n_init=int(r.integers(0, 3)), n_local=int(r.integers(1, 4)), seed=seed)


SEEDS = list(range(101, 113))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_all_stages(seed):
    c = draw_case(seed)
    log("random shape", c)
    B, H_kv, G, S_k, S_q = c["B"], c["H_kv"], c["G"], c["S_k"], c["S_q"]
    topk, n_init, n_local = c["topk"], c["n_init"], c["n_local"]
    H_q, D = H_kv * G, 128
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H_q, S_q, D, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(B, H_kv, S_k, D, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, H_kv, S_k, D, generator=g).to(torch.bfloat16).to(DEV)
    scale = 1 / math.sqrt(D)
    rows = np.arange(S_q)
    if S_q > 400:
        rows = np.unique(np.concatenate([np.arange(70), np.linspace(70, S_q - 71, 150).astype(int),
                                         np.arange(S_q - 70, S_q)]))
    ti = torch.as_tensor(rows, device=DEV)
    qr = sparse_rows_q(q, rows)

    kc, vc = tb.compress_k(k), tb.compress_v(v)
    idx = tb.select_blocks(q, kc, S_k, topk, n_init, n_local)
    out, lse = tb.sparse_attn_fwd(q, k, v, idx, n_init, n_local)
    cmp_out, cmp_lse = tb.compressed_attn_fwd(q, kc, vc, S_k)
    dense_out, dense_lse = tb.dense_attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()

    k64, v64 = np64(k), np64(v)
    kb, kc64 = O.compress_k(k64, BS)
    vb, vc64 = O.compress_v(v64, BS)
    np.testing.assert_array_equal(bits_np(kc), kb)
    np.testing.assert_array_equal(bits_np(vc), vb)

    gidx = idx.cpu().numpy()[:, :, rows]
    if topk > 0:
        ref_idx, scores = O.select_blocks(qr, kc64, S_k, topk, n_init, n_local, BS, scale, rows=rows,
                                          return_scores=True)
        counts = check_selection(gidx, ref_idx, scores, rows, S_q, S_k, topk, n_init, n_local)
        log("  selection rows:", counts)

    ro, rl = O.sparse_attn(qr, k64, v64, gidx, BS, n_init, n_local, scale, rows=rows)
    log("  sparse:", assert_attn_close(out[:, :, ti], lse[:, :, ti], ro, rl, "sparse"))

    co, cl = O.compressed_attn(qr, kc64, vc64, S_k, BS, scale, rows=rows)
    seen = np.isfinite(cl)
    assert not np64(cmp_out[:, :, ti])[~seen].any() and np.all(np64(cmp_lse[:, :, ti])[~seen] == -np.inf)
    if seen.any():
        sm = torch.as_tensor(seen, device=DEV)
        log("  compressed:", assert_attn_close(cmp_out[:, :, ti][sm], cmp_lse[:, :, ti][sm], co[seen], cl[seen],
                                               "compressed"))

    do, dl = O.dense_attn(qr, k64, v64, scale, causal=True, rows=rows)
    log("  dense:", assert_attn_close(dense_out[:, :, ti], dense_lse[:, :, ti], do, dl, "dense"))
