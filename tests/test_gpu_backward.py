"""GPU parity of the block-sparse attention backward against the fp64 oracle.

The GPU computes the four products (S, dP, dQ/dK, dV) with bf16 operands and
fp32 accumulation: P and dS are rounded to bf16 before their products, D is
taken from the bf16 forward output, and each gradient is rounded once to
bf16.  Each term of a gradient sum then carries a relative error of at most
about 2^-8 (two roundings to bf16 of 2^-9 each), so the error of an output
element is bounded by 2^-8 times the same sum taken over absolute values
(the oracle's ``magnitudes``: |dS| replaced by P (|dP| + |D|), which also
covers the error D inherits from the bf16 forward output), plus 2^-9 of the
element for its final rounding.  The test allows 4 x 2^-8 of that magnitude
per row (L2 over the row) and over the whole tensor.  The sums cancel
(dS sums to zero over a row's keys), so the gradients themselves can be much
smaller than these magnitudes; a dropped block or member still moves a row
by about 1/n of its magnitude, n <= 13 here, far above the bound.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.infv2_oracle as O
import trainable_block_sparse_mean_amd as tb
import workloads
from tests.parity import np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAG_REL = 4 * 2.0 ** -8


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rows_close(got, ref, mag, what):
    """got, ref, mag [..., D] float64: per-row and total L2 error against the
    rounding scale of the row."""
    err = np.linalg.norm(got - ref, axis=-1)
    scale = np.maximum(np.linalg.norm(mag, axis=-1), 1e-30)
    rel = err / scale
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape)
    tot = float(np.linalg.norm(got - ref) / max(np.linalg.norm(mag), 1e-30))
    rref = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    log(f"  {what}: worst row err/magnitude {rel.max():.2e} at {worst}, total {tot:.2e} (err/|ref| {rref:.2e})")
    assert rel.max() <= MAG_REL, f"{what}: row {worst} error {rel.max():.3e} of its magnitude"
    assert tot <= MAG_REL, f"{what}: total error {tot:.3e} of the magnitude"


def bf16_randn(shape, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16).to(DEV)


def arbitrary_idx(w, seed):
    """Rows with duplicates, forced blocks, -1 gaps and out-of-causal blocks."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    nb = (w.S_k + 63) // 64
    return torch.randint(-1, nb, (w.B, w.H_kv, w.S_q, w.topk), generator=g, dtype=torch.int32).to(DEV)


def run_case(w, idx_kind, seed=7):
    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    if idx_kind == "select":
        idx = tb.select_blocks(q, tb.compress_k(k), w.S_k, w.topk, w.n_init, w.n_local)
    else:
        idx = arbitrary_idx(w, seed)
    out, lse = tb.sparse_attn_fwd(q, k, v, idx, w.n_init, w.n_local)
    dout = bf16_randn(q.shape, seed + 1)
    dq, dk, dv = tb.sparse_attn_bwd(q, k, v, out, lse, dout, idx, w.n_init, w.n_local)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, idx=idx, out=out, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv)


CASES = [
    ("tiny_g8_select", workloads.TINY.with_(S_q=1024, S_k=1024, topk=4), "select"),
    ("g16_arbitrary", workloads.TINY.with_(H_q=32, H_kv=2, S_q=1536, S_k=1536, topk=6), "arbitrary"),
    ("ragged_sq37_sk1000_b2_g2", workloads.TINY.with_(B=2, H_q=6, H_kv=3, S_q=37, S_k=1000, topk=5), "arbitrary"),
    ("topk0_g4", workloads.TINY.with_(H_q=4, H_kv=1, S_q=700, S_k=700, topk=0), "select"),
    ("g1_no_init", workloads.TINY.with_(H_q=2, H_kv=2, S_q=500, S_k=500, topk=3, n_init=0, n_local=1), "select"),
    ("decode_b2", workloads.TINY.with_(B=2, H_q=16, H_kv=1, S_q=1, S_k=3000, topk=8), "select"),
    ("planted_g16_select", workloads.SWITCH_SPARSE.with_(S_q=2048, S_k=2048, switch_len=0), "select"),
    # long enough that each key block's tokens are split into 2 / 16 pieces summed in a second pass
    ("pieces2_g8", workloads.TINY.with_(S_q=5000, S_k=5000, topk=4), "arbitrary"),
    ("pieces16_g4", workloads.TINY.with_(H_q=4, H_kv=1, S_q=12300, S_k=12300, topk=3), "select"),
    # 16 pieces mapped onto the XCDs with two batches and two KV heads (the piece
    # decode separates them) and arbitrary rows (duplicates, -1, forced blocks)
    ("pieces16_b2_kv2_arbitrary", workloads.TINY.with_(B=2, H_q=8, H_kv=2, S_q=12300, S_k=12300, topk=3),
     "arbitrary"),
    # queries offset into the keys with 2 pieces: the first piece is empty for every block past it
    ("pieces2_offset_sq4200_sk6000", workloads.TINY.with_(H_q=4, H_kv=1, S_q=4200, S_k=6000, topk=5), "arbitrary"),
    # group sizes that are not powers of two (heads >= G of the MFMA columns stay empty)
    ("g3_ragged_sq777_sk900", workloads.TINY.with_(H_q=9, H_kv=3, S_q=777, S_k=900, topk=5, n_init=2, n_local=3),
     "select"),
    ("g7_arbitrary", workloads.TINY.with_(H_q=14, H_kv=2, S_q=600, S_k=600, topk=7), "arbitrary"),
    ("g5_b2", workloads.TINY.with_(B=2, H_q=5, H_kv=1, S_q=1000, S_k=1000, topk=6), "select"),
]


@pytest.mark.parametrize("name,w,idx_kind", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, w, idx_kind):
    log("backward", name, w)
    r = run_case(w, idx_kind)
    dq, dk, dv, mq, mk, mv = O.sparse_attn_bwd(np64(r["q"]), np64(r["k"]), np64(r["v"]), np64(r["dout"]),
                                               r["idx"].cpu().numpy(), 64, w.n_init, w.n_local, 1 / math.sqrt(w.D),
                                               magnitudes=True)
    rows_close(np64(r["dq"]), dq, mq, "dq")
    rows_close(np64(r["dk"]), dk, mk, "dk")
    rows_close(np64(r["dv"]), dv, mv, "dv")
    # keys no query attends get exactly zero
    never = (np.abs(dv).sum(axis=-1) == 0) & (np.abs(dk).sum(axis=-1) == 0)
    assert not np.abs(np64(r["dk"])[never]).any() and not np.abs(np64(r["dv"])[never]).any()


def test_backward_is_bitwise_deterministic():
    w = workloads.TINY.with_(H_q=32, H_kv=2, S_q=2048, S_k=2048, topk=8)
    a = run_case(w, "select")
    b = tb.sparse_attn_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["idx"], w.n_init, w.n_local)
    for x, y, n in zip((a["dq"], a["dk"], a["dv"]), b, ("dq", "dk", "dv")):
        assert torch.equal(x, y), n


@pytest.mark.parametrize("wl", [workloads.LONG_32K], ids=["long_prefill_32k"])
def test_backward_full_size_sampled_rows_and_invariants(wl):
    """At the benchmark size: dq on sampled rows against the oracle (one token
    at a time), and two identities that hold at any size: the key gradients
    of a KV head sum to zero over its keys, and its value gradients sum to the
    output gradients of its heads summed over tokens."""
    log("backward full size", wl)
    r = run_case(wl, "select")
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(wl.S_q, 24, replace=False))
    q64, k64, v64, do64 = (np64(r[n]) for n in ("q", "k", "v", "dout"))
    idx = r["idx"].cpu().numpy()
    G = wl.H_q // wl.H_kv
    ref_rows = np.zeros((wl.B, wl.H_q, rows.size, wl.D))
    mag_rows = np.zeros_like(ref_rows)
    for g in range(wl.H_kv):
        hs = slice(g * G, (g + 1) * G)
        for n, row in enumerate(rows):
            i = wl.S_k - wl.S_q + int(row)
            sel = [int(j) for j in idx[0, g, row] if j >= 0]
            t = O.attend_keys(i, O.forced_blocks(i, 64, wl.n_init, wl.n_local) + sel, 64, wl.S_k)
            parts = O._softmax_attend_grad(q64[0, hs, row], k64[0, g, t], v64[0, g, t], do64[0, hs, row],
                                           1 / math.sqrt(wl.D), magnitudes=True)
            ref_rows[0, hs, n] = parts[0]
            mag_rows[0, hs, n] = parts[3]
    rows_close(np64(r["dq"])[:, :, rows], ref_rows, mag_rows, "dq (sampled rows)")
    dk = r["dk"].float().double()
    dv = r["dv"].float().double()
    dsum_k = dk.sum(dim=2)                                            # [B, H_kv, D]
    scale_k = dk.abs().sum(dim=2)
    assert float((dsum_k.abs() / scale_k.clamp_min(1e-30)).max()) <= 2e-2, "sum of dk over keys is not ~0"
    want_v = r["dout"].float().double().view(wl.B, wl.H_kv, G, wl.S_q, wl.D).sum(dim=(2, 3))
    rel = float((dv.sum(dim=2) - want_v).norm() / want_v.norm())
    log(f"  sum dv vs sum dout: rel {rel:.2e}")
    assert rel <= 1e-2


def test_backward_32k_every_key_against_sampled_tokens():
    """At the benchmark size (16 token pieces per key block, mapped onto the
    XCDs, G = 16): dO is zero except on 256 sampled tokens, so every other
    token contributes exactly zero to every gradient (dP = 0 and D = <dO, O>
    = 0 make dS = 0).  Every element of dK and dV - block 0, which all 32768
    tokens attend, the window blocks and the selected blocks - is compared
    with the oracle's sum over the sampled tokens alone; dQ is compared on the
    sampled rows and must be exactly zero on all others."""
    wl = workloads.LONG_32K
    log("backward 32k, sampled dO", wl)
    x = workloads.make_inputs(wl)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    idx = tb.select_blocks(q, tb.compress_k(k), wl.S_k, wl.topk, wl.n_init, wl.n_local)
    out, lse = tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local)
    rng = np.random.default_rng(9)
    edges = np.linspace(0, wl.S_q, 241).astype(np.int64)
    toks = {int(rng.integers(a, e)) for a, e in zip(edges[:-1], edges[1:])} | {0, 1, 63, 64} | set(range(wl.S_q - 12, wl.S_q))
    toks = np.array(sorted(toks))
    keep = torch.zeros(wl.S_q, dtype=torch.bool, device=DEV)
    keep[torch.as_tensor(toks, device=DEV)] = True
    dout = bf16_randn(q.shape, 21) * keep.view(1, 1, -1, 1).to(torch.bfloat16)
    dq, dk, dv = tb.sparse_attn_bwd(q, k, v, out, lse, dout, idx, wl.n_init, wl.n_local)
    torch.cuda.synchronize()
    log("  gpu done,", toks.size, "tokens with a gradient")
    q64, k64, v64, do64 = (np64(t) for t in (q, k, v, dout))
    idx_np = idx.cpu().numpy()
    G = wl.H_q // wl.H_kv
    scale = 1 / math.sqrt(wl.D)
    ref = [np.zeros((wl.H_q, toks.size, wl.D)), np.zeros(k64.shape[1:]), np.zeros(v64.shape[1:])]
    mag = [np.zeros_like(r) for r in ref]
    for g in range(wl.H_kv):
        hs = slice(g * G, (g + 1) * G)
        for n, row in enumerate(toks):
            i = wl.S_k - wl.S_q + int(row)
            sel = [int(j) for j in idx_np[0, g, row] if j >= 0]
            t = O.attend_keys(i, O.forced_blocks(i, 64, wl.n_init, wl.n_local) + sel, 64, wl.S_k)
            p = O._softmax_attend_grad(q64[0, hs, row], k64[0, g, t], v64[0, g, t], do64[0, hs, row], scale,
                                       magnitudes=True)
            ref[0][hs, n] = p[0]
            mag[0][hs, n] = p[3]
            ref[1][g, t] += p[1]
            ref[2][g, t] += p[2]
            mag[1][g, t] += p[4]
            mag[2][g, t] += p[5]
    dq64 = np64(dq)[0]
    rows_close(dq64[:, toks], ref[0], mag[0], "dq (sampled tokens)")
    others = np.ones(wl.S_q, dtype=bool)
    others[toks] = False
    assert not np.abs(dq64[:, others]).any(), "dq of a token with zero dO is not zero"
    rows_close(np64(dk)[0], ref[1], mag[1], "dk (every key)")
    rows_close(np64(dv)[0], ref[2], mag[2], "dv (every key)")
    # keys no sampled token attends get exactly zero
    never = np.abs(mag[2]).sum(axis=-1) == 0
    log("  keys reached by the sampled tokens:", int((~never).sum()), "of", never.size)
    assert not np.abs(np64(dk)[0][never]).any() and not np.abs(np64(dv)[0][never]).any()
