"""The five workloads at full size on the GPU, checked against the oracle on
sampled query rows (the oracle computes each sampled row on its own), through
the same switch entry point the benchmark times."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.infv2_oracle as O
import trainable_block_sparse_mean_amd as tb
import workloads
from tests.parity import assert_attn_close, check_selection, np64, sparse_rows_q

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sample_rows(S_q, n, rng):
    """Rows spread over the sequence plus both ends and block edges."""
    base = {0, S_q - 1, min(63, S_q - 1), min(64, S_q - 1), S_q // 2}
    base |= set(rng.integers(0, S_q, size=n).tolist())
    return np.array(sorted(base))


def stratified_rows(S_q, n, rng, tail=16):
    """One row drawn in each of n equal strata of the query positions, plus
    the first rows, block edges and the last `tail` rows (the latest window)."""
    edges = np.linspace(0, S_q, n + 1).astype(np.int64)
    pick = {int(rng.integers(a, max(a + 1, e))) for a, e in zip(edges[:-1], edges[1:])}
    pick |= {0, min(63, S_q - 1), min(64, S_q - 1)}
    pick |= set(range(max(0, S_q - tail), S_q))
    return np.array(sorted(pick))


def run_and_check(w, n_rows=24, batches=None, rows=None):
    log("workload", w)
    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    res = tb.attn_fwd(q, k, v, 64, w.topk, w.n_init, w.n_local, w.switch_len, return_idx=True)
    kc = tb.compress_k(k)
    torch.cuda.synchronize()
    log("  gpu done, path", res["path"])
    rng = np.random.default_rng(1)
    rows = sample_rows(w.S_q, n_rows, rng) if rows is None else rows
    bsel = list(range(w.B)) if batches is None else batches
    bt = torch.as_tensor(bsel, device=DEV)
    rt = torch.as_tensor(rows, device=DEV)
    k64, v64 = np64(k[bt]), np64(v[bt])
    q64 = sparse_rows_q(q[bt], rows)
    scale = 1 / math.sqrt(w.D)
    if res["path"] == "dense":
        ro, rl = O.dense_attn(q64, k64, v64, scale, causal=True, rows=rows)
        return assert_attn_close(res["out"][bt][:, :, rt], res["lse"][bt][:, :, rt], ro, rl, w.name), None
    # compression: bit-exact
    ref_bits, _ = O.compress_k(k64, 64)
    kc_np = kc[bt].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(kc_np, ref_bits)
    # selection on the GPU's k_cmp
    ref_idx, scores = O.select_blocks(q64, np64(kc[bt]), w.S_k, w.topk, w.n_init, w.n_local, 64, scale,
                                      rows=rows, return_scores=True)
    gidx = res["blk_idx"][bt][:, :, rt].cpu().numpy()
    counts = check_selection(gidx, ref_idx, scores, rows, w.S_q, w.S_k, w.topk, w.n_init, w.n_local)
    log("  selection rows:", counts)
    # attention on the GPU's selection
    ro, rl = O.sparse_attn(q64, k64, v64, gidx, 64, w.n_init, w.n_local, scale, rows=rows)
    stats = assert_attn_close(res["out"][bt][:, :, rt], res["lse"][bt][:, :, rt], ro, rl, w.name)
    log("  attention:", stats)
    return stats, counts


def test_tiny_prefill_2k():
    run_and_check(workloads.TINY, n_rows=200)


def test_tiny_prefill_2k_literal_prescaled_inputs():
    # literal "scaled by 1/sqrt(128)" inputs: block scores nearly all tie
    # (most rows accepted only under the near-tie rule); attention must match
    stats, counts = run_and_check(workloads.TINY_PRESCALED, n_rows=64)
    log("  near-tie fraction", counts["near_tie"] / max(1, sum(counts.values())))


def test_switch_4k_dense():
    run_and_check(workloads.SWITCH_DENSE, n_rows=16)


def test_switch_8k_sparse():
    run_and_check(workloads.SWITCH_SPARSE, n_rows=32)


def test_long_prefill_32k():
    # 512 strata over the 32768 rows: every stretch of 64 tokens, every candidate
    # count up to 509, and the last window
    w = workloads.LONG_32K
    rows = stratified_rows(w.S_q, 512, np.random.default_rng(11))
    log("  rows", rows.size)
    run_and_check(w, rows=rows)


def test_decode_b16_32k():
    """Every sequence: one query row per KV head takes the fused selection +
    attention launch of the switch entry point."""
    run_and_check(workloads.DECODE_32K, n_rows=1)


def test_extreme_prefill_128k():
    # 512 strata: three quarters of the rows have more than 512 candidates
    # (16 slots per lane in the top-k) and half more than 1024 (32 slots); every
    # row goes through the 32-block-chunk selection kernel (2048 blocks), and
    # the late windows' union lists exceed 1024 entries
    w = workloads.EXTREME_128K
    rows = stratified_rows(w.S_q, 512, np.random.default_rng(12))
    cand = (w.S_k - w.S_q + rows) // 64 - w.n_local - w.n_init + 1
    log("  rows", rows.size, ">512 candidates", int((cand > 512).sum()), ">1024", int((cand > 1024).sum()))
    assert (cand > 1024).sum() >= 200 and (cand > 512).sum() >= 300
    run_and_check(w, rows=rows)
