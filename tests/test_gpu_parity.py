"""GPU (HIP, through the C ABI) vs the fp64 oracle, stage by stage.

Stage isolation: each GPU stage is compared with the oracle run on the GPU's
own output of the previous stage (select on the GPU's k_cmp, attention on
the GPU's blk_idx), so a failure names its stage.  Inputs come from
workloads.py (seeded).  Tolerances are in tests/parity.py.
"""
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


def gpu_inputs(w):
    x = workloads.make_inputs(w)
    return {k: t.to(DEV) for k, t in x.items()}


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------- compress ----

@pytest.mark.parametrize("B,H,S,values", [(1, 2, 4096, "normal"), (2, 1, 1000, "normal"),
                                          (1, 1, 512, "integer"), (1, 1, 63, "normal")])
def test_compress_bit_exact(B, H, S, values):
    w = workloads.TINY.with_(B=B, H_q=H, H_kv=H, S_q=S, S_k=S, values=values)
    log("compress", w)
    x = gpu_inputs(w)
    kc = tb.compress_k(x["k"])
    torch.cuda.synchronize()
    ref_bits, _ = O.compress_k(np64(x["k"]), 64)
    np.testing.assert_array_equal(bits_np(kc), ref_bits)


# --------------------------------------------------------------- select ----

SELECT_CASES = [
    ("tiny_2k_g8", workloads.TINY, None),
    ("switch_4k_g16", workloads.SWITCH_SPARSE.with_(S_q=4096, S_k=4096, switch_len=0), np.arange(0, 4096, 5)),
    ("ragged_sq37_sk3000", workloads.TINY.with_(H_q=32, H_kv=2, S_q=37, S_k=3000, topk=9), None),
    ("g4_topk40", workloads.TINY.with_(H_q=8, H_kv=2, S_q=1500, S_k=1500, topk=40, n_init=2, n_local=3), None),
    # 513-1536 blocks: 8-token workgroups two per CU, one 64-block chunk at a
    # time (ragged last workgroup and chunk; 11 slots per lane in the top-k)
    ("mid_650blk_sq45", workloads.TINY.with_(H_q=32, H_kv=2, S_q=45, S_k=650 * 64 + 17, topk=64), None),
    # 1537-2048 blocks: the same with one 32-block chunk at a time
    ("mid_1700blk_sq30", workloads.TINY.with_(H_q=16, H_kv=1, S_q=30, S_k=1700 * 64 + 5, topk=100, n_init=2), None),
    # past 2048 blocks: the 8-token workgroups (ragged last workgroup), up to
    # 2100 candidates per row (33 slots per lane in the top-k)
    ("wide_2100blk_sq700", workloads.TINY.with_(H_q=32, H_kv=2, S_q=700, S_k=2100 * 64, topk=64), None),
    # the block cap: 4060 candidates per row (64 slots per lane), top-128
    ("cap_4064blk_topk128", workloads.TINY.with_(H_q=16, H_kv=1, S_q=40, S_k=4064 * 64, topk=128), None),
]


@pytest.mark.parametrize("name,w,rows", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_matches_oracle(name, w, rows):
    log("select", name, w)
    x = gpu_inputs(w)
    kc = tb.compress_k(x["k"])
    idx, score = tb.select_blocks(x["q"], kc, w.S_k, w.topk, w.n_init, w.n_local, return_scores=True)
    torch.cuda.synchronize()
    rows = np.arange(w.S_q) if rows is None else rows
    q64 = sparse_rows_q(x["q"], rows)
    ref, scores = O.select_blocks(q64, np64(kc), w.S_k, w.topk, w.n_init, w.n_local, 64,
                                  1 / math.sqrt(w.D), rows=rows, return_scores=True)
    gidx = idx.cpu().numpy()[:, :, rows]
    counts = check_selection(gidx, ref, scores, rows, w.S_q, w.S_k, w.topk, w.n_init, w.n_local)
    log("  selection rows:", counts)
    # the returned scores are the group scores of the kept blocks
    gs = score.cpu().numpy()[:, :, rows]
    for (b, g, r), sig in list(scores.items())[:: max(1, len(scores) // 200)]:
        n = int(np.searchsorted(rows, r))
        sel = gidx[b, g, n]
        for e, j in enumerate(sel):
            if j >= 0:
                assert abs(gs[b, g, n, e] - sig[j]) <= 1e-4 * max(sig[j], 1e-3), (b, g, r, j)
            else:
                assert gs[b, g, n, e] == 0.0
    assert counts["near_tie"] <= 0.02 * sum(counts.values())


def test_select_nonfinite_query_rows_stay_valid():
    """NaN or Inf in a query makes that token's group scores NaN.  Its row must
    still be a valid selection (the top-k keys clear the sign bit, so no row
    can overflow), and every other row must be untouched.  The oracle has no
    defined result for non-finite inputs, so poisoned rows are checked for
    validity only."""
    w = workloads.TINY.with_(H_q=32, H_kv=2, S_q=2048, S_k=2048, topk=12)
    log("select non-finite", w)
    x = gpu_inputs(w)
    q_clean = x["q"].clone()
    nan_rows, inf_rows = [100, 777, 1500, 2047], [300, 1800]
    q = x["q"]
    q[0, 3, nan_rows, 5] = float("nan")    # a head of KV group 0
    q[0, 20, inf_rows, 0] = float("inf")   # a head of KV group 1
    kc = tb.compress_k(x["k"])
    idx = tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local).cpu().numpy()
    for r, g in [(r, 0) for r in nan_rows] + [(r, 1) for r in inf_rows]:
        qb = (w.S_k - w.S_q + r) // 64
        cand = set(range(w.n_init, qb - w.n_local + 1))
        k = min(w.topk, len(cand))
        row = list(idx[0, g, r])
        assert all(j in cand for j in row[:k]) and row[:k] == sorted(set(row[:k])), (r, g, row)
        assert row[k:] == [-1] * (w.topk - k), (r, g, row)
    poisoned = set(nan_rows + inf_rows)
    rows = np.array([r for r in range(0, w.S_q, 3) if r not in poisoned])
    ref, scores = O.select_blocks(sparse_rows_q(q_clean, rows), np64(kc), w.S_k, w.topk, w.n_init, w.n_local, 64,
                                  1 / math.sqrt(w.D), rows=rows, return_scores=True)
    counts = check_selection(idx[:, :, rows], ref, scores, rows, w.S_q, w.S_k, w.topk, w.n_init, w.n_local)
    log("  clean rows:", counts)
    # the other KV group of a poisoned token is untouched too
    for r, g_other in [(r, 1) for r in nan_rows] + [(r, 0) for r in inf_rows]:
        one = np.array([r])
        ref1, sc1 = O.select_blocks(sparse_rows_q(q_clean, one), np64(kc), w.S_k, w.topk, w.n_init, w.n_local, 64,
                                    1 / math.sqrt(w.D), rows=one, return_scores=True)
        check_selection(idx[:, g_other:g_other + 1, one], ref1[:, g_other:g_other + 1], {(0, 0, r): sc1[(0, g_other, r)]},
                        one, w.S_q, w.S_k, w.topk, w.n_init, w.n_local)


def test_select_all_ties_is_bit_exact():
    w = workloads.TINY.with_(H_q=32, H_kv=2, S_q=2048, S_k=2048, topk=12, values="constant_k")
    log("select ties", w)
    x = gpu_inputs(w)
    kc = tb.compress_k(x["k"])
    idx = tb.select_blocks(x["q"], kc, w.S_k, w.topk, w.n_init, w.n_local).cpu().numpy()
    for r in range(w.S_q):
        cand = list(O.candidates(r, 64, w.n_init, w.n_local))
        want = cand[: w.topk] + [-1] * (w.topk - min(w.topk, len(cand)))
        assert list(idx[0, 0, r]) == want and list(idx[0, 1, r]) == want, r


# ------------------------------------------------------ sparse attention ----

SPARSE_CASES = [
    ("tiny_2k_g8", workloads.TINY),
    ("g16_4k_topk16", workloads.SWITCH_SPARSE.with_(S_q=4096, S_k=4096, values="normal")),
    ("ragged_sq37_sk3000", workloads.TINY.with_(H_q=32, H_kv=2, S_q=37, S_k=3000, topk=9)),
    ("ragged_sq1000_sk1000_b2", workloads.TINY.with_(B=2, H_q=6, H_kv=3, S_q=1000, S_k=1000, topk=5)),
    ("topk0", workloads.TINY.with_(S_q=1024, S_k=1024, topk=0)),
    ("g1", workloads.TINY.with_(H_q=2, H_kv=2, S_q=700, S_k=700, topk=3, n_init=0, n_local=1)),
]


@pytest.mark.parametrize("name,w", SPARSE_CASES, ids=[c[0] for c in SPARSE_CASES])
def test_sparse_attention_matches_oracle(name, w):
    log("sparse", name, w)
    x = gpu_inputs(w)
    kc = tb.compress_k(x["k"])
    if w.topk > 0:
        idx = tb.select_blocks(x["q"], kc, w.S_k, w.topk, w.n_init, w.n_local)
    else:
        idx = torch.empty(w.B, w.H_kv, w.S_q, 0, dtype=torch.int32, device=DEV)
    out, lse = tb.sparse_attn_fwd(x["q"], x["k"], x["v"], idx, w.n_init, w.n_local)
    torch.cuda.synchronize()
    rows = np.arange(w.S_q) if w.S_q <= 2048 else np.arange(0, w.S_q, 3)
    q64 = sparse_rows_q(x["q"], rows)
    gidx = idx.cpu().numpy()[:, :, rows]
    ro, rl = O.sparse_attn(q64, np64(x["k"]), np64(x["v"]), gidx, 64, w.n_init, w.n_local,
                           1 / math.sqrt(w.D), rows=rows)
    r = torch.as_tensor(rows, device=DEV)
    stats = assert_attn_close(out[:, :, r], lse[:, :, r], ro, rl, name)
    log("  ", stats)


def test_sparse_attention_arbitrary_indices_duplicates_and_forced():
    # selection rows that repeat blocks, name forced blocks and hold -1 gaps
    w = workloads.TINY.with_(H_q=16, H_kv=1, S_q=900, S_k=900, topk=6)
    log("sparse arbitrary idx", w)
    x = gpu_inputs(w)
    rng = np.random.default_rng(0)
    idx = np.full((1, 1, w.S_q, w.topk), -1, dtype=np.int32)
    for r in range(w.S_q):
        qb = r // 64
        picks = rng.integers(0, qb + 1, size=w.topk)
        picks[rng.random(w.topk) < 0.3] = -1
        idx[0, 0, r] = picks
    out, lse = tb.sparse_attn_fwd(x["q"], x["k"], x["v"], torch.from_numpy(idx).to(DEV), w.n_init, w.n_local)
    torch.cuda.synchronize()
    ro, rl = O.sparse_attn(np64(x["q"]), np64(x["k"]), np64(x["v"]), idx, 64, w.n_init, w.n_local,
                           1 / math.sqrt(128))
    assert_attn_close(out, lse, ro, rl, "arbitrary idx")


def test_sparse_forward_and_backward_at_the_block_cap():
    """4064 key blocks (S_k = 260096), the most the sparse kernels' LDS holds:
    the union list fills the LDS beside the ring.  Queries at the end of the
    keys select blocks across the whole range, the highest ones included."""
    w = workloads.TINY.with_(H_q=16, H_kv=1, S_q=40, S_k=4064 * 64, topk=12)
    log("sparse at the block cap", w)
    x = gpu_inputs(w)
    rng = np.random.default_rng(4)
    idx = np.full((1, 1, w.S_q, w.topk), -1, dtype=np.int32)
    for r in range(w.S_q):
        qb = (w.S_k - w.S_q + r) // 64
        picks = rng.integers(0, qb + 1, size=w.topk)
        picks[:3] = [qb - 2, qb - 3, 2000 + r]
        idx[0, 0, r] = picks
    gidx = torch.from_numpy(idx).to(DEV)
    out, lse = tb.sparse_attn_fwd(x["q"], x["k"], x["v"], gidx, w.n_init, w.n_local)
    dout = torch.randn(x["q"].shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    dq, dk, dv = tb.sparse_attn_bwd(x["q"], x["k"], x["v"], out, lse, dout, gidx, w.n_init, w.n_local)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    q64, k64, v64 = np64(x["q"]), np64(x["k"]), np64(x["v"])
    ro, rl = O.sparse_attn(q64, k64, v64, idx, 64, w.n_init, w.n_local, scale)
    log("  ", assert_attn_close(out, lse, ro, rl, "block cap"))
    rq, rk, rv, mq, mk, mv = O.sparse_attn_bwd(q64, k64, v64, np64(dout), idx, 64, w.n_init, w.n_local, scale,
                                               magnitudes=True)
    for got, ref, mag, n in ((dq, rq, mq, "dq"), (dk, rk, mk, "dk"), (dv, rv, mv, "dv")):
        err = np.linalg.norm(np64(got) - ref, axis=-1)
        lim = 4 * 2.0 ** -8 * np.maximum(np.linalg.norm(mag, axis=-1), 1e-30)
        assert (err <= lim).all(), f"{n}: worst error {float((err / lim).max()):.2f} of the bound"
        assert not np.abs(np64(got)[np.abs(mag).sum(-1) == 0]).any(), f"{n}: unattended rows not zero"


def test_sparse_equals_dense_when_topk_covers_every_block():
    w = workloads.TINY.with_(H_q=32, H_kv=2, S_q=1536, S_k=1536, topk=24)
    log("sparse == dense", w)
    x = gpu_inputs(w)
    kc = tb.compress_k(x["k"])
    idx = tb.select_blocks(x["q"], kc, w.S_k, w.topk, w.n_init, w.n_local)
    so, sl = tb.sparse_attn_fwd(x["q"], x["k"], x["v"], idx, w.n_init, w.n_local)
    do, dl = tb.dense_attn_fwd(x["q"], x["k"], x["v"], causal=True)
    torch.cuda.synchronize()
    # every candidate is selected, so both kernels attend exactly the causal keys
    assert (idx.cpu().numpy()[..., : w.S_q // 64 - 3] >= 0).any()
    rows = np.arange(0, w.S_q, 3)
    ro, rl = O.dense_attn(sparse_rows_q(x["q"], rows), np64(x["k"]), np64(x["v"]), 1 / math.sqrt(128), rows=rows)
    r = torch.as_tensor(rows, device=DEV)
    assert_attn_close(so[:, :, r], sl[:, :, r], ro, rl, "sparse vs dense oracle")
    assert_attn_close(do[:, :, r], dl[:, :, r], ro, rl, "dense vs dense oracle")
    assert float((so.float() - do.float()).abs().max()) <= 1e-2


def test_value_probe_structure():
    # V[t] = one-hot(block(t)): output column j of a head is its attention mass on block j
    w = workloads.TINY.with_(H_q=16, H_kv=1, S_q=4096, S_k=4096, topk=8)
    log("value probe", w)
    x = gpu_inputs(w)
    v = torch.zeros(1, 1, w.S_k, 128)
    v[0, 0, torch.arange(w.S_k), torch.arange(w.S_k) // 64] = 1.0
    v = v.to(torch.bfloat16).to(DEV)
    kc = tb.compress_k(x["k"])
    idx = tb.select_blocks(x["q"], kc, w.S_k, w.topk, w.n_init, w.n_local)
    out, _ = tb.sparse_attn_fwd(x["q"], x["k"], v, idx, w.n_init, w.n_local)
    o = np64(out)[0]
    gi = idx.cpu().numpy()[0, 0]
    for r in range(0, w.S_q, 7):
        qb = r // 64
        want = {0, qb, max(qb - 1, 0)} | {int(j) for j in gi[r] if j >= 0}
        for h in range(16):
            got = set(np.nonzero(o[h, r] > 0)[0].tolist())
            assert got == want, (r, h, sorted(got ^ want))


# ------------------------------------------------------- dense attention ----

DENSE_CASES = [
    ("causal_g16_2k", workloads.TINY.with_(H_q=32, H_kv=2, S_q=2048, S_k=2048), True),
    ("causal_g8_ragged_1000", workloads.TINY.with_(S_q=1000, S_k=1000), True),
    ("bottom_right_sq100_sk1000", workloads.TINY.with_(H_q=16, H_kv=1, S_q=100, S_k=1000), True),
    ("noncausal_sq77_sk300", workloads.TINY.with_(H_q=4, H_kv=2, S_q=77, S_k=300), False),
    ("decode_b4", workloads.TINY.with_(B=4, H_q=32, H_kv=2, S_q=1, S_k=2000), True),
]


@pytest.mark.parametrize("name,w,causal", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_attention_matches_oracle(name, w, causal):
    log("dense", name, w)
    x = gpu_inputs(w)
    out, lse = tb.dense_attn_fwd(x["q"], x["k"], x["v"], causal=causal)
    torch.cuda.synchronize()
    rows = np.arange(w.S_q) if w.S_q <= 1024 else np.arange(0, w.S_q, 4)
    ro, rl = O.dense_attn(sparse_rows_q(x["q"], rows), np64(x["k"]), np64(x["v"]), 1 / math.sqrt(128),
                          causal=causal, rows=rows)
    r = torch.as_tensor(rows, device=DEV)
    log("  ", assert_attn_close(out[:, :, r], lse[:, :, r], ro, rl, name))


# -------------------------------------------------------------- switch ----

@pytest.mark.parametrize("w", [workloads.SWITCH_DENSE, workloads.SWITCH_SPARSE], ids=lambda w: w.name)
def test_switch_and_planted_blocks(w):
    log("switch", w)
    x = gpu_inputs(w)
    res = tb.attn_fwd(x["q"], x["k"], x["v"], 64, w.topk, w.n_init, w.n_local, w.switch_len, return_idx=True)
    torch.cuda.synchronize()
    assert res["path"] == ("dense" if w.S_k <= w.switch_len else "sparse")
    rows = np.arange(0, w.S_q, 61)
    q64 = sparse_rows_q(x["q"], rows)
    ref = O.attention(q64, np64(x["k"]), np64(x["v"]), 64, w.topk, w.n_init, w.n_local, w.switch_len,
                      rows=rows)
    assert ref["path"] == res["path"]
    r = torch.as_tensor(rows, device=DEV)
    if res["path"] == "sparse":
        gidx = res["blk_idx"].cpu().numpy()
        # every token of a planted chunk selects the planted block
        plan = workloads.planted_targets(w)
        for (b, g, c), p in plan.items():
            for rr in (c * 64, c * 64 + 63):
                assert p in set(gidx[b, g, rr].tolist()), (g, c, p)
        # attention parity on the GPU's own selection
        ro, rl = O.sparse_attn(q64, np64(x["k"]), np64(x["v"]), gidx[:, :, rows], 64, w.n_init, w.n_local,
                               1 / math.sqrt(128), rows=rows)
        log("  ", assert_attn_close(res["out"][:, :, r], res["lse"][:, :, r], ro, rl, w.name))
    else:
        log("  ", assert_attn_close(res["out"][:, :, r], res["lse"][:, :, r], ref["out"], ref["lse"], w.name))


def test_switch_boundary_exactly_at_threshold():
    w = workloads.TINY.with_(H_q=32, H_kv=2, S_q=1024, S_k=1024, topk=4)
    x = gpu_inputs(w)
    a = tb.attn_fwd(x["q"], x["k"], x["v"], 64, 4, 1, 2, switch_len=1024)
    d, _ = tb.dense_attn_fwd(x["q"], x["k"], x["v"])
    b = tb.attn_fwd(x["q"], x["k"], x["v"], 64, 4, 1, 2, switch_len=1023)
    torch.cuda.synchronize()
    assert a["path"] == "dense" and torch.equal(a["out"], d)
    assert b["path"] == "sparse" and not torch.equal(b["out"], d)


def test_determinism_bitwise():
    w = workloads.TINY.with_(H_q=32, H_kv=2, S_q=3000, S_k=3000, topk=16)
    x = gpu_inputs(w)
    r1 = tb.attn_fwd(x["q"], x["k"], x["v"], 64, w.topk, 1, 2, 0, return_idx=True)
    r2 = tb.attn_fwd(x["q"], x["k"], x["v"], 64, w.topk, 1, 2, 0, return_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(r1["blk_idx"], r2["blk_idx"])
    assert torch.equal(r1["out"], r2["out"]) and torch.equal(r1["lse"], r2["lse"])


@pytest.mark.parametrize("S_q", [1, 40])
def test_switch_past_2048_blocks(S_q):
    # the whole switch (compress -> selection -> sparse attention) where the
    # selection takes the 8-token workgroups; one query goes there too (the
    # one-query selection kernel stops at 2048 blocks)
    from tests.test_gpu_configs import run_and_check
    w = workloads.TINY.with_(name=f"switch_3000blk_sq{S_q}", H_q=16, H_kv=2, S_q=S_q, S_k=3000 * 64 - 17, topk=64)
    run_and_check(w, rows=np.arange(S_q))
