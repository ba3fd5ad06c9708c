"""GPU decode over a paged, variable-length cache vs the fp64 oracle.

Caches are built the way a server fills them: each sequence's key blocks sit
in pages handed out in a random order.  Pages that no sequence uses, rows past
a sequence's end and unused block-table slots hold noise or out-of-range ids,
so a kernel that reads any of them fails the comparison.  Stage isolation as
in test_gpu_parity: select is checked on the GPU's compressed keys, attention
on the GPU's selection.  Tolerances are in tests/parity.py.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.infv2_oracle as O
import trainable_block_sparse_mean_amd as tb
from tests.parity import assert_attn_close, check_selection, np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BS = 64


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def paged_cache(lens, H_q, H_kv, seed, spare_blocks=2, extra_pages=5):
    """Random paged cache: q [B,H_q,D], k/v pages [P,H_kv,64,D] (bf16, N(0,1)),
    block table [B, max_blocks] (unused slots = 10**9, out of range) and the
    lengths, all on the GPU."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    B, D = len(lens), 128
    nbs = [(L + BS - 1) // BS for L in lens]
    max_blocks = max(nbs) + spare_blocks
    P = sum(nbs) + extra_pages
    order = torch.randperm(P, generator=g)
    table = torch.full((B, max_blocks), 10 ** 9, dtype=torch.int32)
    c = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = order[c:c + nb].to(torch.int32)
        c += nb
    kp = torch.randn(P, H_kv, BS, D, generator=g).to(torch.bfloat16)
    vp = torch.randn(P, H_kv, BS, D, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H_q, D, generator=g).to(torch.bfloat16)
    return dict(q=q.to(DEV), kp=kp.to(DEV), vp=vp.to(DEV), table=table.to(DEV),
                lens=torch.tensor(lens, dtype=torch.int32, device=DEV), max_blocks=max_blocks)


def compressed(c):
    """k_cmp of the cache filled from scratch on the GPU (unwritten rows zero)."""
    B, H_kv = c["table"].shape[0], c["kp"].shape[1]
    k_cmp = torch.zeros(B, H_kv, c["max_blocks"], 128, dtype=torch.bfloat16, device=DEV)
    zeros = torch.zeros_like(c["lens"])
    tb.decode_compress_append(c["kp"], c["table"], zeros, c["lens"], k_cmp, c["max_blocks"])
    return k_cmp


LEN_CASES = [
    ("short_mix", [1, 5, 63, 64, 65, 130], 8, 1, 4),
    ("ragged_g16", [3000, 4160, 1000, 257, 4159, 64 * 40], 32, 2, 16),
    ("g4_topk40", [5000, 2501, 6400], 8, 2, 40),
]


@pytest.mark.parametrize("name,lens,H_q,H_kv,topk", LEN_CASES, ids=[c[0] for c in LEN_CASES])
def test_decode_compress_append_bit_exact(name, lens, H_q, H_kv, topk):
    log("decode compress", name, lens)
    c = paged_cache(lens, H_q, H_kv, seed=11)
    k_cmp = compressed(c)
    torch.cuda.synchronize()
    got = bits_np(k_cmp)
    kp, table = np64(c["kp"]), c["table"].cpu().numpy()
    for b, L in enumerate(lens):
        kb = O.paged_sequence(kp, table[b], L, BS)[None]
        ref, _ = O.compress_k(kb, BS)
        nc = L // BS  # complete blocks only
        np.testing.assert_array_equal(got[b, :, :nc], ref[0, :, :nc])
        assert not got[b, :, nc:].any(), "a row past the complete blocks was written"


def test_decode_compress_append_incremental_equals_from_scratch():
    """Growing every sequence step by step (1 key per step, as in generation,
    and one 100-key jump) gives bitwise the k_cmp of a single fill."""
    lens0 = [60, 63, 64, 127, 500, 1]
    grow = [1, 1, 1, 1, 100, 70]
    c = paged_cache([a + b for a, b in zip(lens0, grow)], 16, 2, seed=12)
    final = c["lens"].clone()
    k_inc = torch.zeros(len(lens0), 2, c["max_blocks"], 128, dtype=torch.bfloat16, device=DEV)
    cur = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    zero = torch.zeros_like(cur)
    tb.decode_compress_append(c["kp"], c["table"], zero, cur, k_inc, c["max_blocks"])
    for step in range(max(grow)):
        nxt = torch.minimum(cur + 1, final)
        tb.decode_compress_append(c["kp"], c["table"], cur, nxt, k_inc, 1)
        cur = nxt
    k_all = compressed(c)
    torch.cuda.synchronize()
    assert torch.equal(k_inc, k_all)


@pytest.mark.parametrize("name,lens,H_q,H_kv,topk", LEN_CASES, ids=[c[0] for c in LEN_CASES])
def test_decode_select_and_attention_match_oracle(name, lens, H_q, H_kv, topk):
    log("decode select+attn", name, lens)
    c = paged_cache(lens, H_q, H_kv, seed=13)
    k_cmp = compressed(c)
    idx, score = tb.decode_select(c["q"], k_cmp, c["lens"], topk, return_scores=True)
    out, lse = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], c["lens"], idx)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    q64, kp, vp = np64(c["q"]), np64(c["kp"]), np64(c["vp"])
    table, kc64, gidx = c["table"].cpu().numpy(), np64(k_cmp), idx.cpu().numpy()
    ref_out = np.zeros((len(lens), H_q, 128))
    ref_lse = np.zeros((len(lens), H_q))
    counts = dict(exact=0, near_tie=0)
    for b, L in enumerate(lens):
        qb = q64[b][None, :, None, :]
        ref_idx, scores = O.select_blocks(qb, kc64[b][None], L, topk, 1, 2, BS, scale, return_scores=True)
        cnt = check_selection(gidx[b][None, :, None, :], ref_idx, scores, [0], 1, L, topk, 1, 2)
        for kk in counts:
            counts[kk] += cnt[kk]
        kb = O.paged_sequence(kp, table[b], L, BS)[None]
        vb = O.paged_sequence(vp, table[b], L, BS)[None]
        ob, lb = O.sparse_attn(qb, kb, vb, gidx[b][None, :, None, :], BS, 1, 2, scale)
        ref_out[b], ref_lse[b] = ob[0, :, 0], lb[0, :, 0]
    log("  selection rows:", counts)
    stats = assert_attn_close(out, lse, ref_out, ref_lse, name)
    log("  attention:", stats)


def test_decode_short_sequences_run_dense():
    """Sequences with at most n_init + n_local + topk blocks attend every key:
    the GPU output equals the oracle's dense attention over the whole cache."""
    lens = [1, 40, 64, 300, 64 * 11]
    topk = 8
    c = paged_cache(lens, 16, 1, seed=14)
    idx = tb.decode_select(c["q"], compressed(c), c["lens"], topk)
    out, lse = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], c["lens"], idx)
    torch.cuda.synchronize()
    kp, vp, table = np64(c["kp"]), np64(c["vp"]), c["table"].cpu().numpy()
    ref_out, ref_lse = np.zeros((len(lens), 16, 128)), np.zeros((len(lens), 16))
    for b, L in enumerate(lens):
        kb = O.paged_sequence(kp, table[b], L, BS)[None]
        vb = O.paged_sequence(vp, table[b], L, BS)[None]
        ob, lb = O.dense_attn(np64(c["q"])[b][None, :, None, :], kb, vb, 1 / math.sqrt(128))
        ref_out[b], ref_lse[b] = ob[0, :, 0], lb[0, :, 0]
    assert_attn_close(out, lse, ref_out, ref_lse, "short sequences")


def test_decode_full_size_b16_32k():
    """The decode benchmark shape (16 sequences, 32 q / 2 kv heads, top-64)
    with lengths around 32k, every sequence checked against the oracle."""
    lens = [32768 - 37 * b for b in range(16)]
    c = paged_cache(lens, 32, 2, seed=15, extra_pages=64)
    k_cmp = compressed(c)
    idx = tb.decode_select(c["q"], k_cmp, c["lens"], 64)
    out, lse = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], c["lens"], idx)
    torch.cuda.synchronize()
    log("decode full size: lengths", lens[0], "..", lens[-1])
    scale = 1 / math.sqrt(128)
    q64, kp, vp = np64(c["q"]), np64(c["kp"]), np64(c["vp"])
    table, kc64, gidx = c["table"].cpu().numpy(), np64(k_cmp), idx.cpu().numpy()
    ref_out, ref_lse = np.zeros((16, 32, 128)), np.zeros((16, 32))
    counts = dict(exact=0, near_tie=0)
    for b, L in enumerate(lens):
        qb = q64[b][None, :, None, :]
        ref_idx, scores = O.select_blocks(qb, kc64[b][None], L, 64, 1, 2, BS, scale, return_scores=True)
        cnt = check_selection(gidx[b][None, :, None, :], ref_idx, scores, [0], 1, L, 64, 1, 2)
        for kk in counts:
            counts[kk] += cnt[kk]
        kb = O.paged_sequence(kp, table[b], L, BS)[None]
        vb = O.paged_sequence(vp, table[b], L, BS)[None]
        ob, lb = O.sparse_attn(qb, kb, vb, gidx[b][None, :, None, :], BS, 1, 2, scale)
        ref_out[b], ref_lse[b] = ob[0, :, 0], lb[0, :, 0]
    log("  selection rows:", counts)
    log("  attention:", assert_attn_close(out, lse, ref_out, ref_lse, "decode b16 32k"))


def test_decode_select_over_512_candidates():
    """Sequences with more than 512 selection candidates take the top-k over
    the whole workgroup (a shared digit histogram instead of one wave's radix
    search); selection checked against the oracle at two top-k sizes."""
    lens = [64 * 520 + 7, 65600, 131072, 100001]
    c = paged_cache(lens, 16, 1, seed=17, spare_blocks=0, extra_pages=3)
    k_cmp = compressed(c)
    scale = 1 / math.sqrt(128)
    q64, kc64 = np64(c["q"]), np64(k_cmp)
    for topk in (64, 250):
        idx = tb.decode_select(c["q"], k_cmp, c["lens"], topk)
        torch.cuda.synchronize()
        gidx = idx.cpu().numpy()
        counts = dict(exact=0, near_tie=0)
        for b, L in enumerate(lens):
            ref_idx, scores = O.select_blocks(q64[b][None, :, None, :], kc64[b][None], L, topk, 1, 2, BS, scale,
                                              return_scores=True)
            cnt = check_selection(gidx[b][None, :, None, :], ref_idx, scores, [0], 1, L, topk, 1, 2)
            for kk in counts:
                counts[kk] += cnt[kk]
        log("  top-%d selection rows:" % topk, counts)


def test_decode_select_ties_over_512_candidates():
    """Equal compressed keys give every candidate the same score: the kept
    blocks are the lowest-index candidates, n_init .. n_init + topk - 1, with
    more than 512 candidates (the whole-workgroup top-k) as with fewer."""
    lens = [64 * 700, 64 * 1500 + 3, 64 * 300]
    c = paged_cache(lens, 16, 1, seed=18, spare_blocks=0)
    c["kp"].zero_()
    idx, score = tb.decode_select(c["q"], compressed(c), c["lens"], 100, return_scores=True)
    torch.cuda.synchronize()
    expect = np.arange(1, 101, dtype=np.int32)
    for b in range(len(lens)):
        assert np.array_equal(idx[b, 0].cpu().numpy(), expect), b
        sc = score[b, 0].cpu().numpy()
        assert np.all(sc == sc[0]) and sc[0] > 0, b


def test_decode_other_forced_blocks():
    """n_init = 0 and a 3-block window (the defaults elsewhere are 1 and 2)."""
    lens = [4000, 129, 2600, 64 * 30 + 1]
    c = paged_cache(lens, 16, 2, seed=16)
    k_cmp = compressed(c)
    idx, score = tb.decode_select(c["q"], k_cmp, c["lens"], 12, n_init=0, n_local=3, return_scores=True)
    out, lse = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], c["lens"], idx, n_init=0, n_local=3)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    q64, kp, vp = np64(c["q"]), np64(c["kp"]), np64(c["vp"])
    table, kc64, gidx = c["table"].cpu().numpy(), np64(k_cmp), idx.cpu().numpy()
    ref_out, ref_lse = np.zeros((len(lens), 16, 128)), np.zeros((len(lens), 16))
    for b, L in enumerate(lens):
        qb = q64[b][None, :, None, :]
        ref_idx, scores = O.select_blocks(qb, kc64[b][None], L, 12, 0, 3, BS, scale, return_scores=True)
        check_selection(gidx[b][None, :, None, :], ref_idx, scores, [0], 1, L, 12, 0, 3)
        kb = O.paged_sequence(kp, table[b], L, BS)[None]
        vb = O.paged_sequence(vp, table[b], L, BS)[None]
        ob, lb = O.sparse_attn(qb, kb, vb, gidx[b][None, :, None, :], BS, 0, 3, scale)
        ref_out[b], ref_lse[b] = ob[0, :, 0], lb[0, :, 0]
    log("  n_init 0, n_local 3:", assert_attn_close(out, lse, ref_out, ref_lse, "decode forced blocks"))


FUSED_CASES = LEN_CASES + [
    ("b16_32k", [32768 - 37 * b for b in range(16)], 32, 2, 64),
    ("over_512_candidates", [64 * 520 + 7, 65600, 131072, 100001], 16, 1, 250),
    ("topk0", [3000, 70, 129], 8, 2, 0),
    # 64 sequences x 2 KV heads: one split per head, the output written directly
    ("b64_one_split", [400 + 23 * b for b in range(64)], 8, 2, 8),
]


@pytest.mark.parametrize("name,lens,H_q,H_kv,topk", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_decode_select_attn_fused_equals_two_calls(name, lens, H_q, H_kv, topk):
    """infv2_decode_select_attn (selection and attention in one launch) gives
    bit for bit the indices, scores, outputs and LSE of infv2_decode_select
    followed by infv2_decode_attn (which the tests above check against the
    oracle), and the same bits again on a second call."""
    log("decode fused", name, lens[:4], "topk", topk)
    c = paged_cache(lens, H_q, H_kv, seed=21, extra_pages=8, spare_blocks=0 if max(lens) > 64 * 2040 else 2)
    k_cmp = compressed(c)
    if topk > 0:
        idx, score = tb.decode_select(c["q"], k_cmp, c["lens"], topk, return_scores=True)
    else:
        idx = torch.empty(len(lens), H_kv, 0, dtype=torch.int32, device=DEV)
    out, lse = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], c["lens"], idx)
    runs = [tb.decode_select_attn(c["q"], k_cmp, c["kp"], c["vp"], c["table"], c["lens"], topk, return_scores=True)
            for _ in range(2)]
    torch.cuda.synchronize()
    for fo, fl, fi, fs in runs:
        assert np.array_equal(bits_np(fo), bits_np(out))
        assert torch.equal(fl, lse)
        if topk > 0:
            assert torch.equal(fi, idx)
            assert torch.equal(fs, score)
    # the other forced blocks; (3, 1) gives sequences shorter than their
    # initial blocks and (2, 5) windows that reach below block 0 (short_mix)
    for ni, nl in ((0, 2), (1, 3), (3, 1), (2, 5)):
        if topk == 0:
            break
        i2 = tb.decode_select(c["q"], k_cmp, c["lens"], topk, n_init=ni, n_local=nl)
        o2, l2 = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], c["lens"], i2, n_init=ni, n_local=nl)
        fo, fl, fi = tb.decode_select_attn(c["q"], k_cmp, c["kp"], c["vp"], c["table"], c["lens"], topk,
                                           n_init=ni, n_local=nl)
        torch.cuda.synchronize()
        assert torch.equal(fi, i2) and torch.equal(fl, l2) and np.array_equal(bits_np(fo), bits_np(o2))
