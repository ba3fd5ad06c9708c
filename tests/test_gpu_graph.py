"""The library's calls inside a captured HIP graph (torch.cuda.graph): a
paged decode step (append, select, attend, branch) and a prefill step
(compress, select, sparse attention), each replayed several times with eager
work and synchronisations between the replays; every replay must equal the
eager result bit for bit (no kernel of these paths uses floating-point
atomics, so they are deterministic)."""
import sys

import pytest
import torch

import trainable_block_sparse_mean_amd as tb
import workloads
from tests.test_gpu_decode import paged_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    return g, outs


def test_decode_step_graph_replays_match_eager():
    lens = [3000, 4097, 129, 64 * 20]
    c = paged_cache(lens, 32, 2, seed=31)
    cur = c["lens"] - 1
    nxt = c["lens"]
    k_cmp = torch.zeros(len(lens), 2, c["max_blocks"], 128, dtype=torch.bfloat16, device=DEV)
    v_cmp = torch.zeros_like(k_cmp)
    zero = torch.zeros_like(cur)
    tb.decode_compress_append(c["kp"], c["table"], zero, cur, k_cmp, c["max_blocks"])
    tb.decode_compress_append(c["vp"], c["table"], zero, cur, v_cmp, c["max_blocks"])

    def step():
        tb.decode_compress_append(c["kp"], c["table"], cur, nxt, k_cmp, 1)
        tb.decode_compress_append(c["vp"], c["table"], cur, nxt, v_cmp, 1)
        idx = tb.decode_select(c["q"], k_cmp, nxt, 16)
        out, lse = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], nxt, idx)
        mixed, _ = tb.decode_compressed_attn(c["q"], k_cmp, v_cmp, nxt, o_sparse=out, w_sparse=0.75, w_cmp=0.25)
        fo, fl, fi = tb.decode_select_attn(c["q"], k_cmp, c["kp"], c["vp"], c["table"], nxt, 16)
        return idx, out, lse, mixed, fo, fl, fi

    eager = [t.clone() for t in step()]
    g, outs = capture(step)
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("idx", "out", "lse", "mixed", "fused out", "fused lse", "fused idx"), outs, eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
        # eager work between replays
        tb.decode_select(c["q"], k_cmp, nxt, 8)
        torch.cuda.synchronize()
    log("decode step: 3 graph replays equal the eager step")


def test_prefill_step_graph_replays_match_eager():
    w = workloads.TINY.with_(H_q=32, H_kv=2, S_q=3000, S_k=3000, topk=12)
    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))

    def step():
        kc = tb.compress_k(k)
        idx = tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local)
        out, lse = tb.sparse_attn_fwd(q, k, v, idx, w.n_init, w.n_local)
        return kc, idx, out, lse

    eager = [t.clone() for t in step()]
    g, outs = capture(step)
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("k_cmp", "idx", "out", "lse"), outs, eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
        tb.dense_attn_fwd(q, k, v)
        torch.cuda.synchronize()
    log("prefill step: 3 graph replays equal the eager step")
