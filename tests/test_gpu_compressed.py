"""GPU compressed-attention branch and the mix of patterns vs the fp64 oracle.

Stage isolation as in test_gpu_parity: the value compression is checked bit
for bit, the branch on the GPU's own compressed keys and values, the mix on
the GPU's own block-sparse output.  Tolerances are in tests/parity.py.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.infv2_oracle as O
import trainable_block_sparse_mean_amd as tb
import workloads
from tests.parity import assert_attn_close, np64, sparse_rows_q
from tests.test_gpu_decode import compressed as decode_k_cmp
from tests.test_gpu_decode import paged_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BS = 64


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("S", [64, 3000, 4096])
def test_compress_v_bit_exact(S):
    log("compress_v S", S)
    w = workloads.TINY.with_(H_kv=2, S_q=S, S_k=S)
    v = workloads.make_inputs(w)["v"]
    got = bits_np(tb.compress_v(v.to(DEV)))
    ref, _ = O.compress_v(np64(v), BS)
    np.testing.assert_array_equal(got, ref)


CASES = [
    ("tiny_2k_g8", workloads.TINY, None),
    ("g16_4k_rows", workloads.LONG_32K.with_(S_q=4096, S_k=4096), np.arange(0, 4096, 5)),
    ("ragged_sq37_sk3000", workloads.TINY.with_(H_q=32, H_kv=2, S_q=37, S_k=3000), None),
    ("first_blocks_sq200", workloads.TINY.with_(H_q=16, H_kv=4, S_q=200, S_k=200), None),
    ("bottom_right_sq2000_sk32k", workloads.LONG_32K.with_(S_q=2000), np.arange(0, 2000, 3)),
]


def _branch_case(w, rows):
    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kc, vc = tb.compress_k(k), tb.compress_v(v)
    rows = np.arange(w.S_q) if rows is None else rows
    return q, k, v, kc, vc, rows


@pytest.mark.parametrize("name,w,rows", CASES, ids=[c[0] for c in CASES])
def test_compressed_branch_matches_oracle(name, w, rows):
    log("compressed branch", name)
    q, _, _, kc, vc, rows = _branch_case(w, rows)
    out, lse = tb.compressed_attn_fwd(q, kc, vc, w.S_k)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(w.D)
    ref, ref_lse = O.compressed_attn(sparse_rows_q(q, rows), np64(kc), np64(vc), w.S_k, BS, scale, rows=rows)
    ti = torch.as_tensor(rows, device=DEV)
    go, gl = out[:, :, ti], lse[:, :, ti]
    seen = np.isfinite(ref_lse)
    # rows that see no block: exactly zero output and an lse of -inf
    assert not np64(go)[~seen].any()
    assert np.all(np64(gl)[~seen] == -np.inf)
    if seen.any():
        stats = assert_attn_close(go[torch.as_tensor(seen, device=DEV)], gl[torch.as_tensor(seen, device=DEV)],
                                  ref[seen], ref_lse[seen], name)
        log("  ", stats, "rows without a visible block:", int((~seen).sum()))


def test_compressed_branch_value_probe_is_exact():
    """Zero keys make every visible compressed key score the same (p = 1
    exactly); values that are one-hot in block index mod 128 make each
    compressed value that one-hot exactly.  A query that sees nv <= 128
    blocks must then output exactly bf16(1/nv) on dims 0 .. nv-1 and 0 on the
    others: the visible set is checked token by token, bit for bit."""
    S, H_kv, G = 64 * 130, 2, 16
    k = torch.zeros(1, H_kv, S, 128, dtype=torch.bfloat16)
    blk = torch.arange(S) // BS
    v = torch.nn.functional.one_hot(blk % 128, 128).to(torch.bfloat16)[None, None].expand(1, H_kv, S, 128)
    q = torch.randn(1, H_kv * G, S, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    q, k, v = q.to(DEV), k.to(DEV), v.contiguous().to(DEV)
    out, lse = tb.compressed_attn_fwd(q, tb.compress_k(k), tb.compress_v(v), S)
    torch.cuda.synchronize()
    rows = torch.arange(64 * 128)                          # nv <= 128 for every one of these rows
    nv = (rows + 1) // BS
    # the kernel scales by the fp32 quotient 1 / nv, then rounds to bf16
    inv = (torch.ones(nv.shape) / nv.clamp(min=1).float())[:, None]
    want = torch.where(torch.arange(128)[None, :] < nv[:, None], inv, torch.zeros(1, 1)).to(torch.bfloat16)
    got = out[0, :, :64 * 128].cpu()
    assert torch.equal(got, want[None].expand_as(got))
    want_lse = torch.where(nv > 0, torch.log(nv.clamp(min=1).float()), torch.tensor(float("-inf")))
    np.testing.assert_allclose(lse[0, :, :64 * 128].cpu().numpy(), want_lse[None].expand(H_kv * G, -1).numpy(),
                               rtol=0, atol=1e-5)


@pytest.mark.parametrize("name,w,rows", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_mix_with_sparse_output(name, w, rows):
    """out = w_sparse * (GPU block-sparse output) + w_cmp * branch, in one
    kernel; also written in place over the sparse output (same bits)."""
    log("mix", name)
    q, k, v, kc, vc, rows = _branch_case(w, rows)
    idx = tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local)
    o_sp, _ = tb.sparse_attn_fwd(q, k, v, idx, w.n_init, w.n_local)
    ws, wc = 0.625, 0.375
    mixed, lse = tb.compressed_attn_fwd(q, kc, vc, w.S_k, o_sparse=o_sp, w_sparse=ws, w_cmp=wc)
    inplace = o_sp.clone()
    tb.compressed_attn_fwd(q, kc, vc, w.S_k, o_sparse=inplace, w_sparse=ws, w_cmp=wc, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(inplace, mixed)
    scale = 1 / math.sqrt(w.D)
    branch, branch_lse = O.compressed_attn(sparse_rows_q(q, rows), np64(kc), np64(vc), w.S_k, BS, scale, rows=rows)
    ti = torch.as_tensor(rows, device=DEV)
    ref = O.mix_patterns([np64(o_sp[:, :, ti]), branch], [ws, wc])
    seen = np.isfinite(branch_lse)
    stats = assert_attn_close(mixed[:, :, ti], None, ref, None, name)
    np.testing.assert_allclose(np64(lse[:, :, ti])[seen], branch_lse[seen], atol=1e-3)
    log("  ", stats)


def test_compressed_branch_at_32k_sampled_rows():
    w = workloads.LONG_32K
    rows = np.unique(np.concatenate([np.arange(0, 130), np.linspace(130, w.S_q - 1, 300).astype(int),
                                     np.arange(w.S_q - 64, w.S_q)]))
    q, _, _, kc, vc, rows = _branch_case(w, rows)
    out, lse = tb.compressed_attn_fwd(q, kc, vc, w.S_k)
    torch.cuda.synchronize()
    ref, ref_lse = O.compressed_attn(sparse_rows_q(q, rows), np64(kc), np64(vc), w.S_k, BS, 1 / math.sqrt(w.D),
                                     rows=rows)
    ti = torch.as_tensor(rows, device=DEV)
    seen = np.isfinite(ref_lse)
    sm = torch.as_tensor(seen, device=DEV)
    log("  32k:", assert_attn_close(out[:, :, ti][sm], lse[:, :, ti][sm], ref[seen], ref_lse[seen], "32k"))
    assert not np64(out[:, :, ti])[~seen].any()


def test_compressed_branch_128k_keys():
    """The last 1024 queries of a 131072-key sequence: 2048 compressed rows,
    32 groups of 64 per window."""
    w = workloads.EXTREME_128K.with_(S_q=1024, values="normal")
    rows = np.arange(0, 1024, 7)
    q, _, _, kc, vc, rows = _branch_case(w, rows)
    out, lse = tb.compressed_attn_fwd(q, kc, vc, w.S_k)
    torch.cuda.synchronize()
    ref, ref_lse = O.compressed_attn(sparse_rows_q(q, rows), np64(kc), np64(vc), w.S_k, BS, 1 / math.sqrt(w.D),
                                     rows=rows)
    ti = torch.as_tensor(rows, device=DEV)
    log("  128k:", assert_attn_close(out[:, :, ti], lse[:, :, ti], ref, ref_lse, "128k"))


DECODE_CASES = [
    ("short_mix", [1, 5, 63, 64, 65, 130], 8, 1),
    ("ragged_g16", [3000, 4160, 1000, 257, 4159, 64 * 40], 32, 2),
    ("b16_32k", [32768 - 37 * b for b in range(16)], 32, 2),
]


@pytest.mark.parametrize("name,lens,H_q,H_kv", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_compressed_branch_and_mix(name, lens, H_q, H_kv):
    """Paged, variable-length decode: the values' compressed rows come from
    the same append call on the value pages; the branch of each sequence's
    query, alone and mixed with its block-sparse output."""
    log("decode compressed", name)
    c = paged_cache(lens, H_q, H_kv, seed=21, extra_pages=8)
    k_cmp = decode_k_cmp(c)
    v_cmp = torch.zeros_like(k_cmp)
    tb.decode_compress_append(c["vp"], c["table"], torch.zeros_like(c["lens"]), c["lens"], v_cmp, c["max_blocks"])
    out, lse = tb.decode_compressed_attn(c["q"], k_cmp, v_cmp, c["lens"])
    idx = tb.decode_select(c["q"], k_cmp, c["lens"], 16)
    o_sp, _ = tb.decode_attn(c["q"], c["kp"], c["vp"], c["table"], c["lens"], idx)
    mixed, _ = tb.decode_compressed_attn(c["q"], k_cmp, v_cmp, c["lens"], o_sparse=o_sp, w_sparse=0.5, w_cmp=0.5)
    torch.cuda.synchronize()
    vp, table = np64(c["vp"]), c["table"].cpu().numpy()
    q64, kc64 = np64(c["q"]), np64(k_cmp)
    ref = np.zeros((len(lens), H_q, 128))
    ref_lse = np.zeros((len(lens), H_q))
    for b, L in enumerate(lens):
        vb = O.paged_sequence(vp, table[b], L, BS)[None]
        _, vc = O.compress_v(vb, BS)
        nc = L // BS
        # the GPU's value rows of the complete blocks are the oracle's, bit for bit
        np.testing.assert_array_equal(bits_np(v_cmp[b, :, :nc]), O.f64_to_bf16(vc[0, :, :nc]))
        o, l = O.compressed_attn(q64[b][None, :, None, :], kc64[b][None], vc, L, BS, 1 / math.sqrt(128))
        ref[b], ref_lse[b] = o[0, :, 0], l[0, :, 0]
    seen = np.isfinite(ref_lse)
    assert not np64(out)[~seen].any() and np.all(np64(lse)[~seen] == -np.inf)
    sm = torch.as_tensor(seen, device=DEV)
    log("  branch:", assert_attn_close(out[sm], lse[sm], ref[seen], ref_lse[seen], name))
    ref_mix = O.mix_patterns([np64(o_sp), ref], [0.5, 0.5])
    log("  mix:", assert_attn_close(mixed, None, ref_mix, None, name + " mix"))


MIX_CASES = CASES[:4] + [("long_32k_rows", workloads.LONG_32K, np.unique(np.concatenate(
    [np.arange(0, 100), np.linspace(100, 32767, 200).astype(int)])))]


@pytest.mark.parametrize("name,w,rows", MIX_CASES, ids=[c[0] for c in MIX_CASES])
def test_mixed_attn_in_one_call_matches_oracle(name, w, rows):
    """infv2_mixed_attn_fwd: w_sparse * sparse + w_cmp * branch against the
    oracle's sparse attention (on the GPU's selection) and branch (on the
    GPU's compressed keys and values).  ragged_sq37 takes the two-call path
    (its block lists are split), the others the fused kernel."""
    log("mixed one call", name)
    q, k, v, kc, vc, rows = _branch_case(w, rows)
    idx = tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local)
    ws_, wc_ = 0.7, 0.3
    out, lse = tb.mixed_attn_fwd(q, k, v, idx, kc, vc, ws_, wc_, w.n_init, w.n_local)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(w.D)
    qr = sparse_rows_q(q, rows)
    ti = torch.as_tensor(rows, device=DEV)
    so, sl = O.sparse_attn(qr, np64(k), np64(v), idx.cpu().numpy()[:, :, rows], BS, w.n_init, w.n_local, scale,
                           rows=rows)
    co, _ = O.compressed_attn(qr, np64(kc), np64(vc), w.S_k, BS, scale, rows=rows)
    ref = O.mix_patterns([so, co], [ws_, wc_])
    log("  ", assert_attn_close(out[:, :, ti], lse[:, :, ti], ref, sl, name))
