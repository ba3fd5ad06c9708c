"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances
----------
* Output O (bf16): max |O_gpu - O_ref| <= 2e-2 and mean |O_gpu - O_ref| <= 2e-3
  (bf16 inputs, fp32 accumulation), plus relative L2 <= 1e-2.
* LSE (fp32): |lse_gpu - lse_ref| <= 1e-3.  Dropping one of ~67 attended
  blocks moves the LSE by about log(67/66) = 0.015, so this sees a missing
  block that the output tolerances cannot.
* Selection: the GPU row must hold exactly min(topk, #candidates) distinct
  ascending candidate indices followed by -1.  It may differ from the oracle's
  row only in blocks whose oracle score lies within 1e-3 (relative) of the
  k-th largest oracle score tau (near-ties); any other difference fails.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.infv2_oracle as O

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
O_REL_L2 = 1e-2
LSE_ABS = 1e-3
NEAR_TIE_REL = 1e-3


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 tensor (any device)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def sparse_rows_q(q: torch.Tensor, rows) -> np.ndarray:
    """float64 [B,H,S_q,D] holding only the given query rows (other rows stay
    zero; np.zeros pages that are never written cost no memory)."""
    B, H, S_q, D = q.shape
    out = np.zeros((B, H, S_q, D))
    rows = np.asarray(rows)
    out[:, :, rows, :] = np64(q[:, :, torch.as_tensor(rows, device=q.device), :])
    return out


def assert_attn_close(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    o = np64(out_gpu)
    diff = np.abs(o - out_ref)
    max_abs, mean_abs = float(diff.max()), float(diff.mean())
    rel_l2 = float(np.linalg.norm(o - out_ref) / max(np.linalg.norm(out_ref), 1e-30))
    msg = f"{what}: max_abs={max_abs:.3e} mean_abs={mean_abs:.3e} rel_l2={rel_l2:.3e}"
    assert max_abs <= O_MAX_ABS and mean_abs <= O_MEAN_ABS and rel_l2 <= O_REL_L2, msg
    if lse_gpu is not None:
        ld = np.abs(np64(lse_gpu) - lse_ref)
        assert float(ld.max()) <= LSE_ABS, f"{what}: lse max diff {float(ld.max()):.3e}"
    return dict(max_abs=max_abs, mean_abs=mean_abs, rel_l2=rel_l2)


def check_selection(gpu_idx: np.ndarray, ref_idx: np.ndarray, scores: dict, rows, S_q: int, S_k: int,
                    topk: int, n_init: int, n_local: int, block_size: int = 64) -> dict:
    """Compare GPU and oracle selections row by row under the near-tie rule.

    gpu_idx, ref_idx: int [B, H_kv, len(rows), topk]; scores: {(b,g,r): sigma}
    from the oracle.  Returns counts; raises AssertionError on a failing row.
    """
    counts = dict(exact=0, near_tie=0)
    off = S_k - S_q
    B, H_kv = ref_idx.shape[:2]
    for b in range(B):
        for g in range(H_kv):
            for n, r in enumerate(rows):
                gr, orow = gpu_idx[b, g, n], ref_idx[b, g, n]
                if np.array_equal(gr, orow):
                    counts["exact"] += 1
                    continue
                i = off + int(r)
                cand = O.candidates(i, block_size, n_init, n_local)
                kk = min(topk, cand.size)
                sel = gr[:kk]
                where = f"(b={b}, g={g}, row={r})"
                assert np.all(gr[kk:] == -1), f"{where}: padding {gr}"
                assert np.all(np.diff(sel) > 0), f"{where}: not ascending/distinct {gr}"
                assert set(sel.tolist()) <= set(cand.tolist()), f"{where}: non-candidate in {gr}"
                sig = scores[(b, g, int(r))]
                tau = np.sort(sig[cand])[::-1][kk - 1]
                diff = set(sel.tolist()) ^ set(int(j) for j in orow[:kk])
                bad = [j for j in diff if abs(sig[j] - tau) > NEAR_TIE_REL * tau]
                assert not bad, f"{where}: blocks {bad} differ beyond the near-tie band (tau={tau})"
                counts["near_tie"] += 1
    return counts
