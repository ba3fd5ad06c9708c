"""Pins of the fp64 oracle to facts outside the oracle itself.

Each test checks the oracle against something it does not compute the same
way: closed forms, library routines on special cases (torch's float->bf16
rounding, scipy's softmax, torch's scaled_dot_product_attention), brute force
written as explicit masks or exhaustive searches, invariants, and a
hand-derived example (tests/golden/scores_hand.json).  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle.infv2_oracle as O
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd_bf16(rng, *shape, scale=1.0):
    """Random bf16-representable float64 values (torch rounding)."""
    x = torch.from_numpy(rng.standard_normal(shape) * scale).float().to(torch.bfloat16)
    return x.double().numpy()


# ---------------------------------------------------------------- bf16 ----

def test_bf16_widening_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x0000, 0x4049], dtype=np.uint16)
    got = O.bf16_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133
    assert np.isinf(got[3]) and got[4] == 0.0
    assert got[5] == 3.140625


def test_bf16_rounding_matches_torch_on_float32_values():
    # for float32 inputs the direct fp64->bf16 rounding equals torch's
    # float32->bf16 round-to-nearest-even (a library routine)
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000),
                        rng.standard_normal(2000) * 1e-38,      # subnormal range
                        rng.standard_normal(2000) * 1e30,
                        (rng.integers(0, 2 ** 16, 4000) / 2 ** 16) + 1.0]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_rounding_hand_cases():
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,                 # exact half -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,             # exact half -> even (1 + 2^-6)
        1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,    # just above half: up (no double rounding)
        -(1.0 + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        2.0 ** -133: 0x0001,                     # smallest subnormal
        2.0 ** -134: 0x0000,                     # half of it -> even (0)
        3 * 2.0 ** -134: 0x0002,                 # 1.5 quanta -> 2
    }
    for x, want in cases.items():
        assert int(O.f64_to_bf16(np.array([x]))[0]) == want, (x, hex(want))


# ------------------------------------------------------------ compress ----

def test_compress_constant_keys_is_identity():
    rng = np.random.default_rng(2)
    row = rnd_bf16(rng, 1, 2, 1, 32)
    k = np.broadcast_to(row, (1, 2, 256, 32)).copy()
    bits, kc = O.compress_k(k, 64)
    assert kc.shape == (1, 2, 4, 32)
    np.testing.assert_array_equal(kc, np.broadcast_to(row, kc.shape))


def test_compress_ramp_closed_form():
    t = np.arange(128, dtype=np.float64)
    k = np.broadcast_to(t[None, None, :, None], (1, 1, 128, 8)).copy()
    _, kc = O.compress_k(k, 64)
    np.testing.assert_array_equal(kc[0, 0, :, 0], [31.5, 95.5])   # means of 0..63, 64..127


def test_compress_tail_zero_padded_divides_by_block_size():
    k = np.ones((1, 1, 100, 4))
    _, kc = O.compress_k(k, 64)
    np.testing.assert_array_equal(kc[0, 0, :, 0], [1.0, 36.0 / 64.0])


def test_compress_rounds_half_to_even():
    k = np.zeros((1, 1, 64, 2))
    k[0, 0, 0, :] = 1.0
    k[0, 0, 1, 0] = 3 * 2.0 ** -8     # mean (1 + 3*2^-8)/64: an exact half
    k[0, 0, 1, 1] = 2.0 ** -9         # mean (1 + 2^-9)/64: below half
    bits, _ = O.compress_k(k, 64)
    assert list(bits[0, 0, 0]) == [0x3C82, 0x3C80]


def test_compress_integer_keys_exact_against_torch_rounding():
    w = workloads.TINY.with_(values="integer", S_q=512, S_k=512)
    k = workloads.make_inputs(w)["k"]
    kf = k.double().numpy()
    bits, _ = O.compress_k(kf, 64)
    # integer sums are exact; /64 is exact; the mean fits float32 exactly
    mean = k.double().reshape(1, 1, 8, 64, 128).sum(3) / 64
    want = mean.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want)


# -------------------------------------------------------------- scores ----

def test_scores_hand_derived_golden():
    gd = json.load(open(os.path.join(GOLDEN, "scores_hand.json")))
    G, D = gd["G"], gd["D"]
    q = np.array(gd["q"], dtype=np.float64).reshape(1, G, 1, D)
    kc = np.log(np.array(gd["k_cmp_log_of"])).reshape(1, 1, -1, D)
    sig = O.group_scores(q, kc, 0, 0, gd["position"], 0, G, gd["scale"], gd["block_size"])
    np.testing.assert_allclose(sig, np.array(gd["sigma_numerators_over_42"]) / 42.0, rtol=1e-14)
    sel = O.select_row(sig, gd["position"], gd["block_size"], gd["topk"], gd["n_init"], gd["n_local"])
    assert list(sel) == gd["selected"]


def test_scores_sum_to_group_size_and_nonnegative():
    rng = np.random.default_rng(3)
    G, D, nb = 4, 16, 20
    q = rnd_bf16(rng, 1, 2 * G, 5, D)
    kc = rnd_bf16(rng, 1, 2, nb, D)
    for i in [63, 64, 100, 500, 1279]:
        for g in range(2):
            sig = O.group_scores(q, kc, 0, g, i, 2, G, 0.25, 64)
            assert sig.size == (i + 1) // 64
            assert np.all(sig >= 0)
            assert abs(sig.sum() - G) < 1e-12


def test_scores_zero_query_uniform():
    G, nb = 3, 9
    q = np.zeros((1, G, 1, 8))
    kc = np.random.default_rng(4).standard_normal((1, 1, nb, 8))
    sig = O.group_scores(q, kc, 0, 0, 64 * 7 + 5, 0, G, 1.0, 64)
    np.testing.assert_allclose(sig, np.full(7, G / 7.0), rtol=1e-14)


def test_scores_single_head_is_causal_softmax_over_compressed_keys():
    rng = np.random.default_rng(5)
    q = rnd_bf16(rng, 1, 1, 1, 32)
    kc = rnd_bf16(rng, 1, 1, 12, 32)
    i = 64 * 9 + 63                      # block 9 complete -> nv = 10
    sig = O.group_scores(q, kc, 0, 0, i, 0, 1, 0.3, 64)
    logits = 0.3 * (kc[0, 0, :10] @ q[0, 0, 0])
    np.testing.assert_allclose(sig, scipy.special.softmax(logits), rtol=1e-13)


def test_scores_ignore_invisible_blocks_and_head_order():
    rng = np.random.default_rng(6)
    G = 4
    q = rnd_bf16(rng, 1, G, 1, 16)
    kc = rnd_bf16(rng, 1, 1, 10, 16)
    i = 64 * 6 + 10                      # nv = 6
    a = O.group_scores(q, kc, 0, 0, i, 0, G, 0.5, 64)
    kc2 = kc.copy()
    kc2[0, 0, 6:] = 100.0                # blocks not yet complete must not matter
    b = O.group_scores(q, kc2, 0, 0, i, 0, G, 0.5, 64)
    np.testing.assert_array_equal(a, b)
    c = O.group_scores(q[:, ::-1].copy(), kc, 0, 0, i, 0, G, 0.5, 64)
    np.testing.assert_allclose(a, c, rtol=1e-14)


def test_scores_one_dominant_block():
    G, D = 2, 4
    q = np.ones((1, G, 1, D))
    kc = np.zeros((1, 1, 8, D))
    kc[0, 0, 3] = 50.0
    sig = O.group_scores(q, kc, 0, 0, 64 * 8 - 1, 0, G, 1.0, 64)
    assert abs(sig[3] - G) < 1e-12 and sig.argmax() == 3


# ------------------------------------------------------------- top-k ----

def test_candidates_closed_form():
    assert list(O.candidates(64 * 10 + 7, 64, 1, 2)) == list(range(1, 9))
    assert O.candidates(64 * 2, 64, 1, 2).size == 0          # qb=2: [1,0] empty
    assert list(O.candidates(64 * 3, 64, 1, 2)) == [1]
    assert list(O.candidates(64 * 3, 64, 0, 1)) == [0, 1, 2]


def _dominates(sig, sel, cand):
    """Every selected candidate beats every unselected one under (sigma desc, index asc)."""
    rest = [c for c in cand if c not in set(sel)]
    return all((sig[a] > sig[b]) or (sig[a] == sig[b] and a < b) for a in sel for b in rest)


def test_select_characterisation_random():
    rng = np.random.default_rng(7)
    for trial in range(200):
        nb = int(rng.integers(1, 40))
        i = 64 * nb + int(rng.integers(0, 64))
        topk = int(rng.integers(0, 12))
        # coarse values force many exact ties
        sig = np.round(rng.random(nb + 1) * 4) / 4
        sel = O.select_row(sig, i, 64, topk, 1, 2)
        cand = list(O.candidates(i, 64, 1, 2))
        chosen = [int(j) for j in sel if j >= 0]
        assert len(chosen) == min(topk, len(cand))
        assert chosen == sorted(chosen) and len(set(chosen)) == len(chosen)
        assert set(chosen) <= set(cand)
        assert all(j == -1 for j in sel[len(chosen):])
        assert _dominates(sig, chosen, cand)


def test_select_exhaustive_tiny():
    # exhaustive search: of all k-subsets, the one with the largest sorted
    # score vector, ties broken by the lexicographically smallest index tuple
    rng = np.random.default_rng(8)
    for trial in range(60):
        nb = int(rng.integers(3, 10))
        i = 64 * nb + 3
        cand = list(O.candidates(i, 64, 1, 2))
        k = int(rng.integers(1, len(cand) + 1)) if cand else 1
        sig = np.round(rng.random(nb + 1) * 3) / 3
        best = None
        for sub in itertools.combinations(cand, min(k, len(cand))):
            key = (sorted((sig[j] for j in sub), reverse=True), [-j for j in sorted(sub)])
            if best is None or key > best[0]:
                best = (key, list(sub))
        sel = [int(j) for j in O.select_row(sig, i, 64, k, 1, 2) if j >= 0]
        assert sel == sorted(best[1])


def test_select_all_ties_takes_lowest_indices():
    w = workloads.TINY.with_(values="constant_k", S_q=1024, S_k=1024, H_q=4, D=32)
    x = workloads.make_inputs(w)
    q, k = x["q"].double().numpy(), x["k"].double().numpy()
    _, kc = O.compress_k(k, 64)
    rows = np.array([0, 200, 511, 700, 1023])
    idx = O.select_blocks(q, kc, 1024, w.topk, w.n_init, w.n_local, 64, 0.1, rows=rows)
    for n, r in enumerate(rows):
        cand = list(O.candidates(int(r), 64, 1, 2))
        want = cand[:w.topk] + [-1] * (w.topk - min(w.topk, len(cand)))
        assert list(idx[0, 0, n]) == want


def test_select_finds_planted_blocks():
    w = workloads.SWITCH_SPARSE.with_(S_q=1024, S_k=1024, H_q=4, H_kv=1, topk=4, switch_len=0)
    x = workloads.make_inputs(w)
    q, k = x["q"].double().numpy(), x["k"].double().numpy()
    _, kc = O.compress_k(k, 64)
    rows = np.arange(0, 1024, 7)
    idx = O.select_blocks(q, kc, 1024, w.topk, w.n_init, w.n_local, 64, 1 / math.sqrt(128), rows=rows)
    plan = workloads.planted_targets(w)
    checked = 0
    for n, r in enumerate(rows):
        c = int(r) // 64
        if (0, 0, c) in plan:
            assert plan[(0, 0, c)] in set(idx[0, 0, n].tolist()), (r, plan[(0, 0, c)])
            checked += 1
    assert checked > 100


# ----------------------------------------------------------- attention ----

def _mask_bruteforce(S_q, S_k, sel_rows, bs, n_init, n_local):
    """Explicit [S_q, S_k] boolean mask: causal AND (initial OR window OR selected)."""
    off = S_k - S_q
    i = off + np.arange(S_q)[:, None]
    t = np.arange(S_k)[None, :]
    blk = t // bs
    qb = i // bs
    m = (blk < n_init) | ((blk <= qb) & (blk > qb - n_local))
    selm = np.zeros((S_q, S_k), dtype=bool)
    for r in range(S_q):
        for j in sel_rows[r]:
            if j >= 0:
                selm[r] |= (blk[0] == j)
    return (m | selm) & (t <= i)


def _masked_attention_bruteforce(q, k, v, mask, scale):
    B, H_q, S_q, D = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    out = np.zeros_like(q)
    lse = np.zeros(q.shape[:3])
    for h in range(H_q):
        z = scale * q[0, h] @ k[0, h // G].T
        z = np.where(mask, z, -np.inf)
        out[0, h] = scipy.special.softmax(z, axis=1) @ v[0, h // G]
        lse[0, h] = scipy.special.logsumexp(z, axis=1)
    return out, lse


@pytest.mark.parametrize("S_q,S_k", [(300, 300), (37, 300), (1, 300)])
def test_sparse_attention_against_explicit_mask(S_q, S_k):
    rng = np.random.default_rng(9)
    G, H_kv, D, bs = 2, 2, 16, 16
    q = rnd_bf16(rng, 1, G * H_kv, S_q, D)
    k = rnd_bf16(rng, 1, H_kv, S_k, D)
    v = rnd_bf16(rng, 1, H_kv, S_k, D)
    nb = (S_k + bs - 1) // bs
    topk = 3
    # arbitrary valid selections, different per KV group
    idx = np.full((1, H_kv, S_q, topk), -1, dtype=np.int32)
    off = S_k - S_q
    for g in range(H_kv):
        for r in range(S_q):
            c = list(O.candidates(off + r, bs, 1, 2))
            pick = sorted(rng.choice(c, size=min(topk, len(c)), replace=False)) if c else []
            idx[0, g, r, :len(pick)] = pick
    out, lse = O.sparse_attn(q, k, v, idx, bs, 1, 2, 0.37)
    for g in range(H_kv):
        mask = _mask_bruteforce(S_q, S_k, idx[0, g], bs, 1, 2)
        o_ref, l_ref = _masked_attention_bruteforce(q[:, g * G:(g + 1) * G], k[:, g:g + 1],
                                                    v[:, g:g + 1], mask, 0.37)
        np.testing.assert_allclose(out[:, g * G:(g + 1) * G], o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, g * G:(g + 1) * G], l_ref, rtol=1e-12, atol=1e-13)
    assert nb > topk + 3


def test_sparse_with_no_selection_is_sink_plus_window():
    rng = np.random.default_rng(10)
    S, D, bs = 200, 8, 16
    q, k, v = (rnd_bf16(rng, 1, 1, S, D) for _ in range(3))
    idx = np.zeros((1, 1, S, 0), dtype=np.int32)
    out, _ = O.sparse_attn(q, k, v, idx, bs, 1, 2, 0.5)
    # textbook mask: first block, plus the current and previous block, causal
    i = np.arange(S)[:, None]
    t = np.arange(S)[None, :]
    mask = ((t < bs) | (t // bs >= i // bs - 1)) & (t <= i)
    o_ref, _ = _masked_attention_bruteforce(q, k, v, mask, 0.5)
    np.testing.assert_allclose(out, o_ref, rtol=1e-12, atol=1e-13)


def test_sparse_equals_dense_when_topk_covers_all_blocks():
    rng = np.random.default_rng(11)
    S, D, bs, G = 256, 16, 16, 2
    q = rnd_bf16(rng, 1, 2 * G, S, D)
    k = rnd_bf16(rng, 1, 2, S, D)
    v = rnd_bf16(rng, 1, 2, S, D)
    _, kc = O.compress_k(k, bs)
    topk = S // bs
    idx = O.select_blocks(q, kc, S, topk, 1, 2, bs, 0.25)
    so, sl = O.sparse_attn(q, k, v, idx, bs, 1, 2, 0.25)
    do, dl = O.dense_attn(q, k, v, 0.25, causal=True)
    np.testing.assert_allclose(so, do, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sl, dl, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("S_q,S_k,causal", [(96, 96, True), (1, 96, True), (40, 96, True), (33, 70, False)])
def test_dense_matches_torch_sdpa_fp64(S_q, S_k, causal):
    rng = np.random.default_rng(12)
    G, H_kv, D = 4, 2, 32
    q = rnd_bf16(rng, 2, G * H_kv, S_q, D)
    k = rnd_bf16(rng, 2, H_kv, S_k, D)
    v = rnd_bf16(rng, 2, H_kv, S_k, D)
    out, lse = O.dense_attn(q, k, v, 0.2, causal=causal)
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(G, dim=1)
    mask = None
    if causal:   # bottom-right aligned
        mask = torch.ones(S_q, S_k, dtype=torch.bool).tril(diagonal=S_k - S_q)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-11, atol=1e-12)
    # lse from the same library: log of the softmax normaliser
    z = 0.2 * (tq @ tk.transpose(-1, -2))
    if mask is not None:
        z = z.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_constant_values_and_zero_query():
    rng = np.random.default_rng(13)
    S, D, bs = 320, 8, 32
    q = rnd_bf16(rng, 1, 2, S, D)
    k = rnd_bf16(rng, 1, 1, S, D)
    v = np.full((1, 1, S, D), 0.75)
    idx = np.full((1, 1, S, 2), -1, dtype=np.int32)
    for r in range(S):
        c = list(O.candidates(r, bs, 1, 2))
        idx[0, 0, r, :min(2, len(c))] = c[-2:] if len(c) >= 2 else c
    out, _ = O.sparse_attn(q, k, v, idx, bs, 1, 2, 0.3)
    np.testing.assert_allclose(out, 0.75, rtol=1e-14)
    # zero query: uniform weights -> mean of attended values, lse = log(count)
    v2 = rnd_bf16(rng, 1, 1, S, D)
    out0, lse0 = O.sparse_attn(np.zeros_like(q), k, v2, idx, bs, 1, 2, 0.3)
    for r in [0, 31, 32, 100, 250, 319]:
        qb = r // bs
        blocks = {0} | {qb, max(qb - 1, 0)} | {int(j) for j in idx[0, 0, r] if j >= 0}
        ts = [t for t in range(r + 1) if t // bs in blocks]
        np.testing.assert_allclose(out0[0, 0, r], v2[0, 0, ts].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(lse0[0, 0, r] - math.log(len(ts))) < 1e-12


def test_attention_value_probe_exposes_attended_blocks():
    # V[t] = one-hot(block(t)): output column j is the attention mass on block j
    rng = np.random.default_rng(14)
    S, bs, nb = 512, 32, 16
    q = rnd_bf16(rng, 1, 2, S, nb)
    k = rnd_bf16(rng, 1, 1, S, nb)
    v = np.zeros((1, 1, S, nb))
    v[0, 0, np.arange(S), np.arange(S) // bs] = 1.0
    _, kc = O.compress_k(k, bs)
    idx = O.select_blocks(q, kc, S, 3, 1, 2, bs, 0.3)
    out, _ = O.sparse_attn(q, k, v, idx, bs, 1, 2, 0.3)
    for r in range(0, S, 5):
        qb = r // bs
        want = {0, qb, max(qb - 1, 0)} | {int(j) for j in idx[0, 0, r] if j >= 0}
        got = set(np.nonzero(out[0, 0, r] > 0)[0].tolist())
        assert got == want, r
        assert abs(out[0, 0, r].sum() - 1.0) < 1e-12


def test_switch_boundary():
    rng = np.random.default_rng(15)
    S, D = 128, 8
    q = rnd_bf16(rng, 1, 2, S, D)
    k = rnd_bf16(rng, 1, 1, S, D)
    v = rnd_bf16(rng, 1, 1, S, D)
    assert O.attention(q, k, v, 16, 2, 1, 2, switch_len=S)["path"] == "dense"
    r = O.attention(q, k, v, 16, 2, 1, 2, switch_len=S - 1)
    assert r["path"] == "sparse" and r["blk_idx"].shape == (1, 1, S, 2)
    d = O.attention(q, k, v, 16, 2, 1, 2, switch_len=S)
    ref, _ = O.dense_attn(q, k, v, 1 / math.sqrt(D))
    np.testing.assert_array_equal(d["out"], ref)


def test_decode_row_is_last_position():
    rng = np.random.default_rng(16)
    S_k, D, bs = 200, 8, 16
    q = rnd_bf16(rng, 1, 2, 1, D)
    k = rnd_bf16(rng, 1, 1, S_k, D)
    v = rnd_bf16(rng, 1, 1, S_k, D)
    full_q = np.zeros((1, 2, S_k, D))
    full_q[:, :, -1] = q[:, :, 0]
    a, la = O.dense_attn(q, k, v, 0.3)
    b, lb = O.dense_attn(full_q, k, v, 0.3, rows=[S_k - 1])
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_scores_group_uses_its_consecutive_heads_only():
    # GQA grouping: query heads g*G .. g*G+G-1 share KV head g
    rng = np.random.default_rng(17)
    G, H_kv, D = 2, 3, 8
    q = rnd_bf16(rng, 1, G * H_kv, 1, D)
    kc = rnd_bf16(rng, 1, H_kv, 6, D)
    i = 64 * 6 - 1
    for g in range(H_kv):
        a = O.group_scores(q, kc, 0, g, i, 0, G, 0.7, 64)
        q2 = q.copy()
        others = [h for h in range(G * H_kv) if h // G != g]
        q2[0, others] = rnd_bf16(rng, len(others), 1, D)
        np.testing.assert_array_equal(O.group_scores(q2, kc, 0, g, i, 0, G, 0.7, 64), a)
        q3 = q.copy()
        q3[0, g * G] = rnd_bf16(rng, 1, D)
        assert not np.array_equal(O.group_scores(q3, kc, 0, g, i, 0, G, 0.7, 64), a)


# --------------------------------------------------- backward (training) ----

def _bwd_case(rng, B=1, G=2, H_kv=2, S=150, D=8, topk=1):
    q = rnd_bf16(rng, B, G * H_kv, S, D)
    k = rnd_bf16(rng, B, H_kv, S, D)
    v = rnd_bf16(rng, B, H_kv, S, D)
    do = rng.standard_normal((B, G * H_kv, S, D))
    # arbitrary selections (duplicates, forced blocks and -1 gaps allowed)
    idx = rng.integers(-1, (S + 63) // 64, size=(B, H_kv, S, topk))
    return q, k, v, do, idx


def test_backward_matches_finite_differences_of_the_forward():
    """Central differences of L = <dO, sparse_attn(q, k, v)>, entry by entry."""
    rng = np.random.default_rng(31)
    q, k, v, do, idx = _bwd_case(rng)
    scale = 0.3
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, 64, 1, 2, scale)

    def loss(q_, k_, v_):
        out, _ = O.sparse_attn(q_, k_, v_, idx, 64, 1, 2, scale)
        return float((out * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            pos = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args_p = dict(q=q, k=k, v=v); args_p[name] = xp
            args_m = dict(q=q, k=k, v=v); args_m[name] = xm
            num = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(num - g[pos]) <= 1e-6 * max(1.0, abs(num)), (name, pos, num, g[pos])


def test_backward_dense_case_matches_torch_autograd_fp64():
    """topk covering every candidate makes the sparse attention dense and
    causal; its gradients then equal torch autograd through SDPA in fp64."""
    rng = np.random.default_rng(32)
    G, H_kv, S, D = 2, 2, 200, 16
    q, k, v, do, _ = _bwd_case(rng, G=G, H_kv=H_kv, S=S, D=D)
    nb = (S + 63) // 64
    idx = np.tile(np.arange(nb), (1, H_kv, S, 1))
    dq, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, 64, 1, 2, 0.25)
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1),
        attn_mask=torch.ones(S, S, dtype=torch.bool).tril(), scale=0.25)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_sum_invariants():
    """Softmax weights sum to one: the key gradients of a KV head sum to zero
    over keys, and its value gradients sum to the output gradients of its
    heads summed over tokens."""
    rng = np.random.default_rng(33)
    G, H_kv = 4, 2
    q, k, v, do, idx = _bwd_case(rng, G=G, H_kv=H_kv, S=300, D=8, topk=2)
    _, dk, dv = O.sparse_attn_bwd(q, k, v, do, idx, 64, 1, 2, 0.3)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    want = do.reshape(1, H_kv, G, 300, 8).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), want, rtol=1e-11, atol=1e-11)



# ---------------------------------------------------------------- decode ----
# A paged cache is defined by scattering each sequence's key blocks into
# pages; the oracle's gather must invert that scatter, and its decode step
# must be the contiguous pipeline run on each sequence with S_q = 1.

def _scatter_into_pages(rng, seqs, bs, extra=3):
    """seqs: list of [H, L_b, D].  Returns (pages [P, H, bs, D], table int32
    [B, max_blocks] with unused slots = -1); pages are handed out in a random
    order and a block's rows past the sequence end stay zero."""
    H, D = seqs[0].shape[0], seqs[0].shape[2]
    nbs = [(s.shape[1] + bs - 1) // bs for s in seqs]
    P = sum(nbs) + extra
    order = rng.permutation(P)
    pages = rng.standard_normal((P, H, bs, D))  # unused pages hold noise
    table = np.full((len(seqs), max(nbs) + 2), -1, dtype=np.int32)
    c = 0
    for b, s in enumerate(seqs):
        for j in range(nbs[b]):
            p = int(order[c])
            c += 1
            table[b, j] = p
            rows = s[:, j * bs:(j + 1) * bs, :]
            pages[p] = 0.0
            pages[p, :, :rows.shape[1], :] = rows
    return pages, table


def test_paged_sequence_inverts_the_page_scatter():
    rng = np.random.default_rng(31)
    bs = 8
    lens = [1, 7, 8, 9, 40, 23]
    seqs = [rng.standard_normal((2, L, 4)) for L in lens]
    pages, table = _scatter_into_pages(rng, seqs, bs)
    for b, s in enumerate(seqs):
        np.testing.assert_array_equal(O.paged_sequence(pages, table[b], lens[b], bs), s)


def test_decode_paged_equals_per_sequence_pipeline():
    rng = np.random.default_rng(32)
    bs, H_kv, G, D, topk = 64, 2, 2, 8, 3
    lens = [1, 64, 65, 300, 900, 640]
    ks = [rng.standard_normal((H_kv, L, D)) for L in lens]
    vs = [rng.standard_normal((H_kv, L, D)) for L in lens]
    kp, table = _scatter_into_pages(rng, ks, bs)
    vp = np.zeros_like(kp)
    for b, v in enumerate(vs):  # the values take the same pages as the keys
        for j in range((lens[b] + bs - 1) // bs):
            rows = v[:, j * bs:(j + 1) * bs, :]
            vp[table[b, j], :, :rows.shape[1], :] = rows
    q = rng.standard_normal((len(lens), H_kv * G, D))
    kcs, idx, out, lse = O.decode_paged(q, kp, vp, table, np.array(lens), bs, topk, 1, 2, 0.4)
    for b, L in enumerate(lens):
        qb = q[b][None, :, None, :]
        _, kc = O.compress_k(ks[b][None], bs)
        np.testing.assert_array_equal(kcs[b], kc[0])
        ib = O.select_blocks(qb, kc, L, topk, 1, 2, bs, 0.4)
        np.testing.assert_array_equal(idx[b], ib[0, :, 0])
        ob, lb = O.sparse_attn(qb, ks[b][None], vs[b][None], ib, bs, 1, 2, 0.4)
        np.testing.assert_array_equal(out[b], ob[0, :, 0])
        np.testing.assert_array_equal(lse[b], lb[0, :, 0])


def test_decode_short_sequence_is_dense_softmax():
    """A sequence with no more than n_init + n_local + topk blocks attends all
    of its keys: the output is the plain softmax over them."""
    rng = np.random.default_rng(33)
    bs, H_kv, G, D, topk = 64, 1, 4, 8, 2
    lens = [5, 64, 200, 320]  # at most 1 + 2 + 2 = 5 blocks
    ks = [rng.standard_normal((H_kv, L, D)) for L in lens]
    vs = [rng.standard_normal((H_kv, L, D)) for L in lens]
    kp, table = _scatter_into_pages(rng, ks, bs)
    vp = np.zeros_like(kp)
    for b, v in enumerate(vs):
        for j in range((lens[b] + bs - 1) // bs):
            rows = v[:, j * bs:(j + 1) * bs, :]
            vp[table[b, j], :, :rows.shape[1], :] = rows
    q = rng.standard_normal((len(lens), H_kv * G, D))
    _, _, out, lse = O.decode_paged(q, kp, vp, table, np.array(lens), bs, topk, 1, 2, 0.3)
    for b in range(len(lens)):
        for h in range(H_kv * G):
            z = 0.3 * ks[b][h // G] @ q[b, h]
            np.testing.assert_allclose(out[b, h], scipy.special.softmax(z) @ vs[b][h // G], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], scipy.special.logsumexp(z), rtol=1e-12)


# ------------------------------------------------------- approximate LSE ----

def test_strided_lse_stride_one_is_the_exact_score():
    rng = np.random.default_rng(41)
    q = rng.standard_normal((1, 4, 3, 8))
    kc = rng.standard_normal((1, 2, 40, 8))
    for i in (63, 64, 700, 2559):
        np.testing.assert_allclose(O.group_scores_strided_lse(q, kc, 0, 1, i, 2, 2, 0.7, 64, 1),
                                   O.group_scores(q, kc, 0, 1, i, 2, 2, 0.7, 64), rtol=1e-13, atol=1e-16)


def test_strided_lse_is_exact_when_each_group_shares_one_key():
    """If the R blocks of every group have the same compressed key, a group's
    sample times its visible count is its exact sum: the approximate scores
    equal the exact ones, also for a last group cut short."""
    rng = np.random.default_rng(42)
    R = 4
    base = rng.standard_normal((1, 2, 10, 8))
    kc = np.repeat(base, R, axis=2)                     # 40 blocks, groups of 4 equal keys
    q = rng.standard_normal((1, 4, 1, 8))
    for i in (64 * 37 - 1, 64 * 40 - 1, 64 * 9 + 5):    # nv = 37 (last group 1 of 4), 40, 9
        np.testing.assert_allclose(O.group_scores_strided_lse(q, kc, 0, 0, i, 0, 2, 0.5, 64, R),
                                   O.group_scores(q, kc, 0, 0, i, 0, 2, 0.5, 64), rtol=1e-13, atol=1e-15)


def test_strided_lse_hand_case():
    """One head, nv = 5, stride 2: samples are blocks 0, 2, 4 standing for 2,
    2 and 1 blocks, so LSE = log(2 e^z0 + 2 e^z2 + e^z4)."""
    q = np.zeros((1, 1, 1, 2))
    q[0, 0, 0] = [1.0, 0.0]
    kc = np.zeros((1, 1, 5, 2))
    kc[0, 0, :, 0] = [0.5, -1.0, 2.0, 0.25, -0.5]       # z_j = scale * k_j0 with scale 1
    sig = O.group_scores_strided_lse(q, kc, 0, 0, 64 * 5 - 1, 0, 1, 1.0, 64, 2)
    z = kc[0, 0, :, 0]
    lse = math.log(2 * math.exp(z[0]) + 2 * math.exp(z[2]) + math.exp(z[4]))
    np.testing.assert_allclose(sig, np.exp(z - lse), rtol=1e-14)



def test_strided_select_stride_one_is_select_blocks():
    """Stride 1 samples every block with weight 1, so the selection is the
    exact one bit for bit: two batches and two KV heads, queries that end
    before the keys (position i = S_k - S_q + r), distinct n_init and n_local,
    a row subset, ragged last block."""
    rng = np.random.default_rng(43)
    B, H_kv, G, S_q, S_k, D = 2, 2, 3, 70, 64 * 11 + 9, 8
    q = rng.standard_normal((B, H_kv * G, S_q, D))
    kc = rng.standard_normal((B, H_kv, (S_k + 63) // 64, D))
    rows = np.array([0, 3, 31, 40, 69])
    for topk, n_init, n_local in ((3, 2, 3), (5, 1, 2), (9, 0, 1)):
        exact = O.select_blocks(q, kc, S_k, topk, n_init, n_local, 64, 0.4, rows=rows)
        strided = O.select_blocks_strided_lse(q, kc, S_k, topk, n_init, n_local, 64, 0.4, 1, rows=rows)
        assert exact.dtype == strided.dtype and np.array_equal(exact, strided)


def test_strided_select_hand_case_flips_a_choice():
    """Two heads, one KV group, query at position 383 (nv = 6 visible blocks,
    candidates 1 .. 4 with n_init = n_local = 1), top-1, scale 1, scores
    z_1 = (0, 2, 0, 0, 0, 0) and z_2 = (0, 0, 2.2, 0, 0, 0).
    Exact: L_1 = log(e^2 + 5) = 2.5168, L_2 = log(e^2.2 + 5) = 2.6408, so
    sigma_1 = e^(2-L_1) + e^(-L_2) = 0.6677 < sigma_2 = e^(-L_1) + e^(2.2-L_2)
    = 0.7242: block 2.  Stride 2 samples blocks 0, 2, 4 for two blocks each:
    L_1 = log 6 = 1.7918 (block 1 unseen), L_2 = log(4 + 2 e^2.2) = 3.0933,
    so sigma_1 = 1.2767 > sigma_2 = 0.5760: block 1."""
    q = np.zeros((1, 2, 1, 2))
    q[0, 0, 0] = [1.0, 0.0]
    q[0, 1, 0] = [0.0, 1.0]
    kc = np.zeros((1, 1, 6, 2))
    kc[0, 0, 1, 0] = 2.0
    kc[0, 0, 2, 1] = 2.2
    S_k = 384
    exact = O.select_blocks(q, kc, S_k, 1, 1, 1, 64, 1.0)
    strided = O.select_blocks_strided_lse(q, kc, S_k, 1, 1, 1, 64, 1.0, 2)
    assert exact[0, 0, 0, 0] == 2 and strided[0, 0, 0, 0] == 1
    # the scores behind the two choices, from the closed forms above
    sig_e = O.group_scores(q, kc, 0, 0, 383, 0, 2, 1.0, 64)
    sig_s = O.group_scores_strided_lse(q, kc, 0, 0, 383, 0, 2, 1.0, 64, 2)
    L1, L2 = math.log(math.e ** 2 + 5), math.log(math.e ** 2.2 + 5)
    np.testing.assert_allclose(sig_e[1:3], [math.exp(2 - L1) + math.exp(-L2), math.exp(-L1) + math.exp(2.2 - L2)],
                               rtol=1e-13)
    L1s, L2s = math.log(6.0), math.log(4 + 2 * math.e ** 2.2)
    np.testing.assert_allclose(sig_s[1:3], [math.exp(2 - L1s) + math.exp(-L2s), math.exp(-L1s) + math.exp(2.2 - L2s)],
                               rtol=1e-13)

# ------------------------------------------------ compressed-attention branch ----

def test_compressed_attn_zero_keys_average_the_visible_blocks():
    """With all keys zero every compressed key scores the same, so each query
    averages the compressed values of the blocks it sees.  V is constant in
    each block (bf16 values), so that average is the plain mean of V over the
    first 64 * nv tokens: pins nv = floor((i+1)/64) and that the values, not
    the keys, are averaged."""
    rng = np.random.default_rng(51)
    B, H_kv, G, S, D = 1, 2, 2, 64 * 6 + 17, 8
    per_block = rnd_bf16(rng, B, H_kv, 7, D)
    v = np.repeat(per_block, 64, axis=2)[:, :, :S]
    k = np.zeros((B, H_kv, S, D))
    _, kc = O.compress_k(k, 64)
    _, vc = O.compress_v(np.repeat(per_block, 64, axis=2), 64)
    q = rnd_bf16(rng, B, H_kv * G, S, D)
    out, lse = O.compressed_attn(q, kc, vc, S, 64, 0.5)
    for i in range(S):
        nv = (i + 1) // 64
        for h in range(H_kv * G):
            if nv == 0:
                assert not out[0, h, i].any() and lse[0, h, i] == -np.inf
                continue
            np.testing.assert_allclose(out[0, h, i], v[0, h // G, :64 * nv].mean(axis=0), rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse[0, h, i], math.log(nv), rtol=1e-13)


@pytest.mark.parametrize("S_q,S_k", [(200, 200), (70, 333), (1, 640)])
def test_compressed_attn_matches_sdpa_with_block_end_positions(S_q, S_k):
    """Compressed key j stands at the position of its block's last token
    (64 j + 63): a query sees it iff that position is at or before its own,
    the textbook causal mask over those positions.  torch's SDPA in fp64
    with that mask (bottom-right aligned queries) on the rows that see at
    least one block; the others are zero with lse -inf."""
    rng = np.random.default_rng(52)
    B, H_kv, G, D = 2, 2, 4, 16
    nb = (S_k + 63) // 64
    q = rnd_bf16(rng, B, H_kv * G, S_q, D)
    kc = rnd_bf16(rng, B, H_kv, nb, D)
    vc = rnd_bf16(rng, B, H_kv, nb, D)
    out, lse = O.compressed_attn(q, kc, vc, S_k, 64, 0.3)
    pos = torch.arange(S_q) + (S_k - S_q)
    mask = (64 * torch.arange(nb) + 63)[None, :] <= pos[:, None]          # [S_q, nb]
    seen = mask.any(dim=1).numpy()
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(kc).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(vc).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3).numpy()
    z = (0.3 * (tq @ tk.transpose(-1, -2))).masked_fill(~mask, float("-inf"))
    ref_lse = torch.logsumexp(z, dim=-1).numpy()
    np.testing.assert_allclose(out[:, :, seen], ref[:, :, seen], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, seen], ref_lse[:, :, seen], rtol=1e-12)
    assert not out[:, :, ~seen].any() and np.all(lse[:, :, ~seen] == -np.inf)


def test_compressed_attn_single_head_weights_are_the_block_scores():
    """With one head per group the selection score of a block is that head's
    softmax weight over the visible compressed keys, so the branch output is
    the score-weighted sum of the compressed values."""
    rng = np.random.default_rng(53)
    q = rnd_bf16(rng, 1, 3, 50, 32)
    kc = rnd_bf16(rng, 1, 3, 9, 32)
    vc = rnd_bf16(rng, 1, 3, 9, 32)
    S_k = 64 * 9
    out, _ = O.compressed_attn(q, kc, vc, S_k, 64, 0.4)
    off = S_k - 50
    for h in range(3):
        for r in (0, 17, 49):
            sig = O.group_scores(q, kc, 0, h, off + r, r, 1, 0.4, 64)
            np.testing.assert_allclose(out[0, h, r], sig @ vc[0, h, :sig.size], rtol=1e-12, atol=1e-14)


def test_compressed_attn_last_query_is_the_unmasked_softmax():
    """The last token of a sequence of whole blocks sees every block: there
    the causal branch is the sketch's unmasked softmax over all compressed
    keys (scipy's softmax)."""
    rng = np.random.default_rng(54)
    q = rnd_bf16(rng, 1, 2, 1, 16)
    kc = rnd_bf16(rng, 1, 1, 11, 16)
    vc = rnd_bf16(rng, 1, 1, 11, 16)
    out, lse = O.compressed_attn(q, kc, vc, 64 * 11, 64, 0.25)
    for h in range(2):
        z = 0.25 * kc[0, 0] @ q[0, h, 0]
        np.testing.assert_allclose(out[0, h, 0], scipy.special.softmax(z) @ vc[0, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[0, h, 0], scipy.special.logsumexp(z), rtol=1e-13)


def test_compressed_attn_constant_values():
    rng = np.random.default_rng(55)
    q = rnd_bf16(rng, 1, 4, 130, 8)
    kc = rnd_bf16(rng, 1, 2, 3, 8)
    vc = np.full((1, 2, 3, 8), -1.75)
    out, _ = O.compressed_attn(q, kc, vc, 130, 64, 1.0)
    np.testing.assert_array_equal(out[:, :, :63], 0.0)
    np.testing.assert_allclose(out[:, :, 63:], -1.75, rtol=1e-14)


def test_mix_patterns_closed_forms():
    rng = np.random.default_rng(56)
    a, b = rng.standard_normal((2, 3, 5, 8)), rng.standard_normal((2, 3, 5, 8))
    np.testing.assert_array_equal(O.mix_patterns([a, b], [1.0, 0.0]), a)
    np.testing.assert_array_equal(O.mix_patterns([a, b], [0.0, 1.0]), b)
    np.testing.assert_allclose(O.mix_patterns([a, b], [0.25, 0.75]), 0.25 * a + 0.75 * b, rtol=1e-15)
    c = np.full((2, 3, 5, 8), 3.0)
    np.testing.assert_allclose(O.mix_patterns([c, -c, c], [0.5, 0.25, 0.125]), 3.0 * 0.375, rtol=1e-15)
