"""The allocation-free switch (infv2_attn_fwd_noalloc) through the C ABI,
against infv2_attn_fwd on the same inputs: outputs, LSE and selected blocks
bit for bit on calls in a row that reuse the library's fixed scratch - the
32768-token workload (17 MB of the 32 MiB scratch), then a smaller ragged
shape that reads only what it wrote itself, then a dense-path shape."""
import sys

import pytest
import torch

import trainable_block_sparse_mean_amd as tb
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_both(w, switch_len):
    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    ref = tb.attn_fwd(q, k, v, 64, w.topk, w.n_init, w.n_local, switch_len, return_idx=True)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H_q, w.S_q, dtype=torch.float32, device=DEV)
    idx = torch.full((w.B, w.H_kv, w.S_q, w.topk), -7, dtype=torch.int32, device=DEV) if w.topk else None
    tb.attn_fwd_noalloc(q, k, v, out, lse, idx if ref["path"] == "sparse" else None, 64, w.topk, w.n_init,
                        w.n_local, switch_len)
    torch.cuda.synchronize()
    assert torch.equal(out, ref["out"]), "out"
    assert torch.equal(lse, ref["lse"]), "lse"
    if ref["path"] == "sparse" and w.topk:
        assert torch.equal(idx, ref["blk_idx"]), "blk_idx"
    return ref["path"]


def test_noalloc_switch_equals_workspace_switch_on_calls_in_a_row():
    big = workloads.LONG_32K
    small = workloads.TINY.with_(H_q=8, H_kv=2, S_q=1300, S_k=3000, topk=9)
    dense = workloads.TINY.with_(H_q=16, H_kv=2, S_q=777, S_k=777, topk=4)
    for w, sl in ((big, 0), (small, 0), (dense, 4096), (small, 0)):
        log("noalloc vs workspace switch:", w.name, w.B, w.H_q, w.H_kv, w.S_q, w.S_k, "switch_len", sl)
        path = run_both(w, sl)
        log("  path", path, "bitwise equal")
