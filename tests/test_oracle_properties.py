"""Randomised invariants of the fp64 oracle over many small shapes (CPU).

hypothesis draws the shapes and the seed; each property holds for every
input by the definitions the oracle follows, so a plausible slip (an
off-by-one in visibility, a wrong candidate range, a dropped normalisation)
fails on some draw.
"""
import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle.infv2_oracle as O

BS = 64
SHAPES = st.fixed_dictionaries({
    "G": st.integers(1, 4), "H_kv": st.integers(1, 2), "S_k": st.integers(1, 640),
    "frac": st.floats(0.0, 1.0), "topk": st.integers(0, 6), "n_init": st.integers(0, 2),
    "n_local": st.integers(1, 3), "seed": st.integers(0, 2 ** 31 - 1)})


def draw(c, D=8):
    rng = np.random.default_rng(c["seed"])
    S_q = max(1, int(round(c["frac"] * c["S_k"])))
    q = rng.standard_normal((1, c["G"] * c["H_kv"], S_q, D))
    k = rng.standard_normal((1, c["H_kv"], c["S_k"], D))
    v = rng.standard_normal((1, c["H_kv"], c["S_k"], D))
    return q, k, v, S_q


@settings(max_examples=40, deadline=None)
@given(SHAPES)
def test_selection_is_a_valid_top_k(c):
    q, k, _, S_q = draw(c)
    _, kc = O.compress_k(k, BS)
    idx, scores = O.select_blocks(q, kc, c["S_k"], c["topk"], c["n_init"], c["n_local"], BS, 0.5,
                                  return_scores=True)
    off = c["S_k"] - S_q
    for (b, g, r), sig in scores.items():
        i = off + r
        cand = O.candidates(i, BS, c["n_init"], c["n_local"])
        row = idx[b, g, r]
        kk = min(c["topk"], cand.size)
        sel = row[:kk]
        assert np.all(row[kk:] == -1)
        assert np.all(np.diff(sel) > 0) and set(sel.tolist()) <= set(cand.tolist())
        # every kept block scores at least as high as every dropped candidate;
        # an equal score is kept only at a lower index
        dropped = sorted(set(cand.tolist()) - set(sel.tolist()))
        for j in sel:
            for d in dropped:
                assert sig[j] > sig[d] or (sig[j] == sig[d] and j < d)
        # group scores: non-negative, summing to G over the visible blocks
        nv = O.visible_blocks(i, BS)
        if nv:
            assert np.all(sig >= 0) and abs(sig.sum() - c["G"]) <= 1e-9 * c["G"]


@settings(max_examples=30, deadline=None)
@given(SHAPES)
def test_attention_outputs_are_convex_combinations_of_attended_values(c):
    q, k, v, S_q = draw(c)
    _, kc = O.compress_k(k, BS)
    idx = O.select_blocks(q, kc, c["S_k"], c["topk"], c["n_init"], c["n_local"], BS, 0.5)
    out, lse = O.sparse_attn(q, k, v, idx, BS, c["n_init"], c["n_local"], 0.5)
    off = c["S_k"] - S_q
    G = c["G"]
    for g in range(c["H_kv"]):
        for r in range(S_q):
            i = off + r
            sel = [int(j) for j in idx[0, g, r] if j >= 0]
            t = O.attend_keys(i, O.forced_blocks(i, BS, c["n_init"], c["n_local"]) + sel, BS, c["S_k"])
            assert t.size >= 1 and t.max() <= i and i in t  # causal, own key always attended
            vv = v[0, g, t]
            for h in range(g * G, (g + 1) * G):
                assert np.all(out[0, h, r] <= vv.max(axis=0) + 1e-12)
                assert np.all(out[0, h, r] >= vv.min(axis=0) - 1e-12)
                # the log-sum-exp bounds: max logit <= lse <= max logit + log(#keys)
                z = 0.5 * (k[0, g, t] @ q[0, h, r])
                assert z.max() - 1e-12 <= lse[0, h, r] <= z.max() + math.log(t.size) + 1e-12


@settings(max_examples=30, deadline=None)
@given(SHAPES)
def test_compressed_branch_is_a_convex_combination_of_visible_block_means(c):
    q, k, v, S_q = draw(c)
    _, kc = O.compress_k(k, BS)
    _, vc = O.compress_v(v, BS)
    out, lse = O.compressed_attn(q, kc, vc, c["S_k"], BS, 0.5)
    off = c["S_k"] - S_q
    G = c["G"]
    for g in range(c["H_kv"]):
        for r in range(S_q):
            nv = O.visible_blocks(off + r, BS)
            for h in range(g * G, (g + 1) * G):
                if nv == 0:
                    assert not out[0, h, r].any() and lse[0, h, r] == -np.inf
                    continue
                rows = vc[0, g, :nv]
                assert np.all(out[0, h, r] <= rows.max(axis=0) + 1e-12)
                assert np.all(out[0, h, r] >= rows.min(axis=0) - 1e-12)
                assert np.isfinite(lse[0, h, r]) and lse[0, h, r] <= 0.5 * np.abs(kc[0, g, :nv] @ q[0, h, r]).max() + math.log(nv) + 1e-12
