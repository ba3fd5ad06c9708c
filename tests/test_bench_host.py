"""Host-side logic of bench.py: the closed-form count of attended keys that
the algorithmic FLOP figures use, checked against the oracle's attended sets."""
import numpy as np
import pytest

import bench
import oracle.infv2_oracle as O


@pytest.mark.parametrize("S_q,S_k,topk,n_init,n_local", [(700, 700, 5, 1, 2), (37, 3000, 9, 1, 2),
                                                         (300, 300, 0, 0, 1), (500, 500, 40, 2, 3),
                                                         (1, 4000, 64, 1, 2)])
def test_attended_keys_closed_form(S_q, S_k, topk, n_init, n_local):
    keys = bench.attended_keys(S_q, S_k, 64, topk, n_init, n_local)
    off = S_k - S_q
    for r in range(0, S_q, max(1, S_q // 97)):
        i = off + r
        cand = list(O.candidates(i, 64, n_init, n_local))
        sel = cand[:topk]                      # any k' candidates: the count does not depend on which
        want = O.attend_keys(i, O.forced_blocks(i, 64, n_init, n_local) + sel, 64, S_k).size
        assert keys[r] == want, (r, keys[r], want)


def test_flop_counts_of_the_long_prefill_workload():
    import workloads
    sparse, dense, select, _ = bench.flop_counts(workloads.LONG_32K)
    assert dense == 4 * 128 * 32 * (32768 * 32769 // 2)
    assert abs(sparse / 2.137e12 - 1) < 1e-3 and abs(dense / sparse - 4.12) < 0.01
