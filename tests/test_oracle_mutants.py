"""Planted mistakes in the oracle must make a pin fail (CPU only).

Each mutant replaces one oracle function with a plausible wrong version (a
dropped term, an off-by-one index, a flipped tie rule, a wrong head mapping)
and runs the pins that should catch it.  The real oracle is restored after
each case by monkeypatch.
"""
import numpy as np
import pytest

import oracle.infv2_oracle as impl
import tests.test_oracle_pins as pins


def _scores_no_normalisation(q, k_cmp, b, g, i, r, G, scale, block_size):
    nv = impl.visible_blocks(i, block_size)
    qh = q[b, g * G:(g + 1) * G, r, :]
    return np.exp(scale * (qh @ k_cmp[b, g, :nv, :].T)).sum(axis=0)


def _scores_wrong_head(q, k_cmp, b, g, i, r, G, scale, block_size):
    nv = impl.visible_blocks(i, block_size)
    if nv == 0:
        return np.zeros(0)
    qh = q[b, g::max(q.shape[1] // G, 1), r, :][:G]       # strided instead of consecutive heads
    z = scale * (qh @ k_cmp[b, g, :nv, :].T)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return p.sum(0)


def _visible_off_by_one(i, block_size):
    return i // block_size


def _select_ties_high(sigma, i, block_size, topk, n_init, n_local):
    c = impl.candidates(i, block_size, n_init, n_local)
    out = np.full(topk, -1, dtype=np.int32)
    if topk == 0 or c.size == 0:
        return out
    order = np.lexsort((-c, -sigma[c]))
    chosen = np.sort(c[order[:min(topk, c.size)]])
    out[:chosen.size] = chosen
    return out


def _forced_window_short(i, block_size, n_init, n_local):
    qb = i // block_size
    f = set(range(0, min(n_init, qb + 1)))
    f.update(range(max(qb - n_local + 2, 0), qb + 1))
    return sorted(f)


def _compress_divide_by_count(k, block_size):
    B, H, S, D = k.shape
    nb = (S + block_size - 1) // block_size
    out = np.zeros((B, H, nb, D))
    for j in range(nb):
        out[:, :, j] = k[:, :, j * block_size:(j + 1) * block_size].mean(axis=2)
    bits = impl.f64_to_bf16(out)
    return bits, impl.bf16_to_f64(bits)


def _bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _softmax_attend_no_max_in_lse(qh, kk, vv, scale):
    z = scale * (qh @ kk.T)
    zmax = z.max(axis=1, keepdims=True)
    w = np.exp(z - zmax)
    l = w.sum(axis=1, keepdims=True)
    return (w / l) @ vv, np.log(l)[:, 0]


def _grad_no_rowsum_term(qh, kk, vv, do, scale, magnitudes=False):
    z = scale * (qh @ kk.T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dz = p * (do @ vv.T)                                   # softmax Jacobian without -<dO, o>
    return scale * (dz @ kk), scale * (dz.T @ qh), p.T @ do


def _grad_dk_unscaled(qh, kk, vv, do, scale, magnitudes=False):
    dq, dk, dv = impl.__dict__["_real_grad"](qh, kk, vv, do, scale)
    return dq, dk / scale, dv


def _grad_dv_unnormalised(qh, kk, vv, do, scale, magnitudes=False):
    dq, dk, _ = impl.__dict__["_real_grad"](qh, kk, vv, do, scale)
    z = scale * (qh @ kk.T)
    return dq, dk, np.exp(z - z.max(axis=1, keepdims=True)).T @ do


def _paged_blocks_reversed(pages, table_row, length, block_size):
    nb = (length + block_size - 1) // block_size
    blocks = [pages[int(table_row[j])] for j in reversed(range(nb))]
    return np.concatenate(blocks, axis=1)[:, :length, :]


def _paged_drops_last_key(pages, table_row, length, block_size):
    return impl.__dict__["_real_paged"](pages, table_row, max(length - 1, 1), block_size)


def _strided_unweighted(q, k_cmp, b, g, i, r, G, scale, block_size, stride):
    nv = impl.visible_blocks(i, block_size)
    qh = q[b, g * G:(g + 1) * G, r, :]
    z = scale * (qh @ k_cmp[b, g, :nv, :].T)
    zs = z[:, ::stride]                                  # samples not weighted by their group size
    lse = np.log(np.exp(zs).sum(axis=1, keepdims=True))
    return np.exp(z - lse).sum(axis=0)


def _strided_select_swaps_init_local(q, k_cmp, S_k, topk, n_init, n_local, block_size, scale, stride, rows=None,
                                     return_scores=False):
    return impl.__dict__["_real_strided_select"](q, k_cmp, S_k, topk, n_local, n_init, block_size, scale, stride,
                                                 rows, return_scores)


def _strided_select_row_as_position(q, k_cmp, S_k, topk, n_init, n_local, block_size, scale, stride, rows=None,
                                    return_scores=False):
    # takes query row r to sit at key position r (ignores S_k - S_q)
    return impl.__dict__["_real_strided_select"](q, k_cmp, q.shape[2], topk, n_init, n_local, block_size, scale,
                                                 stride, rows, return_scores)


def _strided_select_exact_lse(q, k_cmp, S_k, topk, n_init, n_local, block_size, scale, stride, rows=None,
                              return_scores=False):
    return impl.select_blocks(q, k_cmp, S_k, topk, n_init, n_local, block_size, scale, rows, return_scores)


def _cmp_unmasked(q, k_cmp, v_cmp, S_k, block_size, scale, rows=None):
    nb = k_cmp.shape[2]
    return impl.__dict__["_real_cmp"](q, k_cmp, v_cmp, nb * block_size + q.shape[2] - 1, block_size, scale, rows)


def _cmp_sees_own_block(q, k_cmp, v_cmp, S_k, block_size, scale, rows=None):
    # counts the block holding the query as visible (floor(i/BS) + 1 blocks)
    return impl.__dict__["_real_cmp"](q, k_cmp, v_cmp, min(S_k + block_size - 1, k_cmp.shape[2] * block_size),
                                      block_size, scale, rows)


def _cmp_values_from_keys(q, k_cmp, v_cmp, S_k, block_size, scale, rows=None):
    return impl.__dict__["_real_cmp"](q, k_cmp, k_cmp, S_k, block_size, scale, rows)


def _mix_unweighted(outputs, weights):
    return sum(np.asarray(o, dtype=np.float64) for o in outputs)


MUTANTS = [
    ("group_scores", _scores_no_normalisation, [pins.test_scores_sum_to_group_size_and_nonnegative,
                                                pins.test_scores_hand_derived_golden]),
    ("group_scores", _scores_wrong_head, [pins.test_scores_group_uses_its_consecutive_heads_only]),
    ("visible_blocks", _visible_off_by_one, [pins.test_scores_single_head_is_causal_softmax_over_compressed_keys]),
    ("select_row", _select_ties_high, [pins.test_select_exhaustive_tiny,
                                       pins.test_select_characterisation_random]),
    ("forced_blocks", _forced_window_short, [pins.test_sparse_with_no_selection_is_sink_plus_window]),
    ("compress_k", _compress_divide_by_count, [pins.test_compress_tail_zero_padded_divides_by_block_size]),
    ("f64_to_bf16", _bf16_truncate, [pins.test_bf16_rounding_hand_cases]),
    ("_softmax_attend", _softmax_attend_no_max_in_lse, [pins.test_dense_matches_torch_sdpa_fp64]),
    ("_softmax_attend_grad", _grad_no_rowsum_term, [pins.test_backward_sum_invariants,
                                                    pins.test_backward_dense_case_matches_torch_autograd_fp64]),
    ("_softmax_attend_grad", _grad_dk_unscaled, [pins.test_backward_matches_finite_differences_of_the_forward,
                                                 pins.test_backward_dense_case_matches_torch_autograd_fp64]),
    ("_softmax_attend_grad", _grad_dv_unnormalised, [pins.test_backward_sum_invariants,
                                                     pins.test_backward_dense_case_matches_torch_autograd_fp64]),
    ("group_scores_strided_lse", _strided_unweighted, [pins.test_strided_lse_is_exact_when_each_group_shares_one_key,
                                                       pins.test_strided_lse_hand_case]),
    ("select_blocks_strided_lse", _strided_select_swaps_init_local, [pins.test_strided_select_stride_one_is_select_blocks]),
    ("select_blocks_strided_lse", _strided_select_row_as_position, [pins.test_strided_select_stride_one_is_select_blocks]),
    ("select_blocks_strided_lse", _strided_select_exact_lse, [pins.test_strided_select_hand_case_flips_a_choice]),
    ("compressed_attn", _cmp_unmasked, [pins.test_compressed_attn_zero_keys_average_the_visible_blocks]),
    ("compressed_attn", _cmp_sees_own_block, [pins.test_compressed_attn_zero_keys_average_the_visible_blocks,
                                              pins.test_compressed_attn_constant_values]),
    ("compressed_attn", _cmp_values_from_keys, [pins.test_compressed_attn_zero_keys_average_the_visible_blocks,
                                                pins.test_compressed_attn_single_head_weights_are_the_block_scores]),
    ("mix_patterns", _mix_unweighted, [pins.test_mix_patterns_closed_forms]),
    ("paged_sequence", _paged_blocks_reversed, [pins.test_paged_sequence_inverts_the_page_scatter,
                                                pins.test_decode_paged_equals_per_sequence_pipeline]),
    ("paged_sequence", _paged_drops_last_key, [pins.test_paged_sequence_inverts_the_page_scatter,
                                               pins.test_decode_short_sequence_is_dense_softmax]),
]


@pytest.mark.parametrize("name,mutant,catchers", MUTANTS, ids=[m[0] + ":" + m[1].__name__ for m in MUTANTS])
def test_pin_catches_mutant(monkeypatch, name, mutant, catchers):
    monkeypatch.setattr(impl, "_real_grad", impl._softmax_attend_grad, raising=False)
    monkeypatch.setattr(impl, "_real_paged", impl.paged_sequence, raising=False)
    monkeypatch.setattr(impl, "_real_cmp", impl.compressed_attn, raising=False)
    monkeypatch.setattr(impl, "_real_strided_select", impl.select_blocks_strided_lse, raising=False)
    monkeypatch.setattr(impl, name, mutant)
    for pin in catchers:
        with pytest.raises(AssertionError):
            if pin is pins.test_dense_matches_torch_sdpa_fp64:
                pin(96, 96, True)
            else:
                pin()
