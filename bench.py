"""Benchmark of the InfLLM-V2 sparse attention forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole sparse path on one batch resident in HBM: key
compression -> group-summed block selection + top-k -> block-sparse attention
(the dense/sparse switch entry point with the sequence above the switch
length).  Default workload: long prefill, batch 1, 32768 tokens, 32 query /
2 KV heads, head dim 128, block 64, top-64 + 1 initial + 2 sliding blocks.

Prints ONE JSON line.  `value` is the effective attention throughput of the
step: algorithmic attention FLOPs (4*D per query head and attended key) per
second.  Per-stage times come from HIP events on the stream the kernels run
on.  `roofline` describes the dominant kernel (the block-sparse attention);
`cpu_baseline` times the fp64 oracle on a bounded sample of query rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_fwd_long_prefill_32k_traffic.json")
ATTN_SOURCES = [os.path.join(ROOT, "trainable_block_sparse_mean_amd", "csrc", f)
                for f in ("attn.hip", "attn_common.hpp", "common.hpp", "kernels.hpp")]


def attended_keys(S_q, S_k, bs, topk, n_init, n_local):
    """Keys attended by each query row (closed form of the attended set)."""
    import numpy as np
    i = (S_k - S_q) + np.arange(S_q, dtype=np.int64)
    qb = i // bs
    diag = i - bs * qb + 1
    init = np.minimum(n_init, qb)                      # initial blocks below qb
    win_lo = np.maximum(qb - n_local + 1, 0)           # window blocks below qb: win_lo .. qb-1
    win = qb - win_lo
    overlap = np.maximum(0, np.minimum(init, qb) - win_lo)   # initial blocks inside the window
    n_cand = np.maximum(0, qb - n_local - n_init + 1)
    sel = np.minimum(topk, n_cand)
    return diag + bs * (init + win - overlap + sel)


def flop_counts(w):
    import numpy as np
    keys = attended_keys(w.S_q, w.S_k, w.block_size, w.topk, w.n_init, w.n_local)
    sparse = 4.0 * w.D * w.H_q * w.B * float(keys.sum())
    i = (w.S_k - w.S_q) + np.arange(w.S_q, dtype=np.int64)
    dense = 4.0 * w.D * w.H_q * w.B * float((i + 1).sum())
    select = 2 * 2.0 * w.D * w.H_q * w.B * float(((i + 1) // w.block_size).sum())
    return sparse, dense, select, keys


def source_hash():
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when the kernel sources changed since the counters were taken."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256") != source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def blas_threads():
    """Threads the oracle's BLAS calls use."""
    try:
        import threadpoolctl
        return max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(w, x, target_s=15.0):
    """The fp64 oracle, as it is, on a bounded sample of query rows."""
    import numpy as np
    import oracle.infv2_oracle as O
    threads = blas_threads()
    q, k, v = (x[n] for n in ("q", "k", "v"))
    t0 = time.perf_counter()
    k64 = k.double().numpy()
    v64 = v.double().numpy()
    _, kc = O.compress_k(k64, w.block_size)
    t_compress = time.perf_counter() - t0
    scale = 1 / math.sqrt(w.D)
    keys = attended_keys(w.S_q, w.S_k, w.block_size, w.topk, w.n_init, w.n_local)
    done_rows, flops, t_rows = 0, 0.0, 0.0
    n = 8
    rng = np.random.default_rng(0)
    while t_rows < target_s:
        rows = np.sort(rng.choice(w.S_q, size=n, replace=False))
        q64 = np.zeros((w.B, w.H_q, w.S_q, w.D))
        q64[:, :, rows, :] = q[:, :, rows, :].double().numpy()
        t1 = time.perf_counter()
        idx = O.select_blocks(q64, kc, w.S_k, w.topk, w.n_init, w.n_local, w.block_size, scale, rows=rows)
        O.sparse_attn(q64, k64, v64, idx, w.block_size, w.n_init, w.n_local, scale, rows=rows)
        t_rows += time.perf_counter() - t1
        done_rows += n
        flops += 4.0 * w.D * w.H_q * w.B * float(keys[rows].sum())
        n = min(2 * n, 512)
    # whole-step estimate: compression once + the per-row cost of every row
    total_rows = w.S_q
    step_s = t_compress + t_rows * total_rows / done_rows
    sparse_flops = 4.0 * w.D * w.H_q * w.B * float(keys.sum())
    return dict(value=sparse_flops / step_s / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=(f"{done_rows} random query rows (both KV groups) of {w.name}: select + attend "
                        f"timed {t_rows:.1f} s, plus full key compression {t_compress:.2f} s; "
                        f"scaled to all {total_rows} rows"),
                step_s_estimate=step_s)


def dist(ms):
    """Median, 10th and 90th percentile of per-call times (ms)."""
    a = sorted(ms)
    pick = lambda f: a[min(len(a) - 1, int(round(f * (len(a) - 1))))]
    return {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4), "calls": len(a)}


def measured_gemm_tflops(torch, dev, n=8192, reps=10):
    """bf16 GEMM throughput of the installed BLAS (torch.matmul, n x n x n):
    the practical MFMA ceiling the kernels are also set against."""
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    c1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 / (c0.elapsed_time(c1) / reps * 1e-3) / 1e12


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def seeded_dout(q, torch):
    """A seeded gradient of the attention output (bf16, N(0,1))."""
    g = torch.Generator(device="cpu")
    g.manual_seed(17)
    return torch.randn(*q.shape, generator=g).to(torch.bfloat16).to(q.device)


def time_decode_paged(torch, tb, workloads, dev, reps=50):
    """One generation step of the decode workload (16 sequences, 32 q / 2 kv
    heads, top-64) over a paged cache: append the compressed key of any block
    the new token completes, then select and attend in one launch (also timed
    as separate selection and attention calls).  The 16 sequences hold 32768 - 37 b
    keys (ragged) in 64-key pages handed out in a random order.  Returns
    {paged step ms, its parts, the contiguous path's step at one length}."""
    wl = workloads.DECODE_32K
    g = torch.Generator(device="cpu")
    g.manual_seed(23)
    B, H_q, H_kv, D = wl.B, wl.H_q, wl.H_kv, wl.D
    lens = [wl.S_k - 37 * b for b in range(B)]
    nbs = [(L + 63) // 64 for L in lens]
    max_blocks = max(nbs) + 1
    P = sum(nbs) + B
    order = torch.randperm(P, generator=g)
    table = torch.zeros(B, max_blocks, dtype=torch.int32)
    c = 0
    for b in range(B):  # every sequence owns nbs[b] + 1 pages (room for the next block)
        table[b, :nbs[b] + 1] = order[c:c + nbs[b] + 1].to(torch.int32)
        c += nbs[b] + 1
    kp = torch.randn(P, H_kv, 64, D, generator=g).to(torch.bfloat16).to(dev)
    vp = torch.randn(P, H_kv, 64, D, generator=g).to(torch.bfloat16).to(dev)
    q = torch.randn(B, H_q, D, generator=g).to(torch.bfloat16).to(dev)
    table = table.to(dev)
    cur = torch.tensor(lens, dtype=torch.int32, device=dev)
    nxt = cur + 1
    k_cmp = torch.zeros(B, H_kv, max_blocks, D, dtype=torch.bfloat16, device=dev)
    tb.decode_compress_append(kp, table, torch.zeros_like(cur), cur, k_cmp, max_blocks)

    def step():  # selection and attention in one launch (infv2_decode_select_attn)
        tb.decode_compress_append(kp, table, cur, nxt, k_cmp, 1)
        return tb.decode_select_attn(q, k_cmp, kp, vp, table, nxt, wl.topk, wl.n_init, wl.n_local)

    def step_three_calls():  # the same step through the separate selection and attention calls
        tb.decode_compress_append(kp, table, cur, nxt, k_cmp, 1)
        idx = tb.decode_select(q, k_cmp, nxt, wl.topk, wl.n_init, wl.n_local)
        return tb.decode_attn(q, kp, vp, table, nxt, idx, wl.n_init, wl.n_local)

    def timed(f, n):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # the same step captured once as a HIP graph and replayed: a decode step is
    # a chain of small launches, which a graph issues without per-launch host work
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph_ms = timed(graph.replay, reps)
    except RuntimeError as e:  # report, do not fail the benchmark line
        graph_ms = f"capture failed: {e}"

    res = {"paged_step_ms": timed(step, reps),
           "paged_step_three_calls_ms": timed(step_three_calls, reps),
           "append_ms": timed(lambda: tb.decode_compress_append(kp, table, cur, nxt, k_cmp, 1), reps)}
    idx = tb.decode_select(q, k_cmp, nxt, wl.topk, wl.n_init, wl.n_local)
    res["select_ms"] = timed(lambda: tb.decode_select(q, k_cmp, nxt, wl.topk, wl.n_init, wl.n_local), reps)
    res["attn_ms"] = timed(lambda: tb.decode_attn(q, kp, vp, table, nxt, idx, wl.n_init, wl.n_local), reps)
    res["select_attn_fused_ms"] = timed(
        lambda: tb.decode_select_attn(q, k_cmp, kp, vp, table, nxt, wl.topk, wl.n_init, wl.n_local), reps)
    # the contiguous path at one length (every sequence 32768 keys): it
    # compresses the whole cache each step
    x = workloads.make_inputs(wl)
    qc, kc, vc = (x[n].to(dev) for n in ("q", "k", "v"))
    plan = tb.AttnPlan(wl.B, wl.H_q, wl.H_kv, wl.S_q, wl.S_k, wl.D, wl.block_size, wl.topk, wl.n_init,
                       wl.n_local, 0, None, dev)
    res["contiguous_step_ms"] = timed(lambda: plan.run(qc, kc, vc), reps)
    res = {k: round(v, 4) for k, v in res.items()}
    res["paged_step_graph_ms"] = round(graph_ms, 4) if isinstance(graph_ms, float) else graph_ms
    # HBM roofline of the step: the K and V rows of the attended blocks (the
    # last block holds only the sequence's tail), the compressed keys selection
    # scores, and Q, O
    per = wl.topk + wl.n_init + wl.n_local
    kv = 0
    for L in [n + 1 for n in lens]:
        nb = (L + 63) // 64
        blocks = min(nb, per)
        kv += ((blocks - 1) * 64 + (L - 64 * (nb - 1))) * H_kv * D * 2 * 2
    kcmp = sum((n + 1) // 64 for n in lens) * H_kv * D * 2
    qo = 2 * B * H_q * D * 2
    res["hbm_roofline"] = {"attn_bytes": kv + qo, "attn_tbs": round((kv + qo) / (res["attn_ms"] * 1e-3) / 1e12, 3),
                           "attn_frac": round((kv + qo) / (res["attn_ms"] * 1e-3) / 8e12, 4),
                           "step_bytes": kv + kcmp + qo,
                           "step_ideal_ms": round((kv + kcmp + qo) / 8e12 * 1e3, 4),
                           "step_frac": round((kv + kcmp + qo) / (res["paged_step_ms"] * 1e-3) / 8e12, 4),
                           "peak_tbs": 8.0}
    return res


def shared_selection(torch, w, frac, dev, seed=7):
    """Block indices of the workload's shape in which the 16 tokens of each
    query window share round(frac * topk) of their selected blocks, the rest
    drawn per token: every row gets min(topk, candidates) distinct candidate
    blocks (n_init .. qb - n_local), ascending, -1 padded, so it attends as
    many keys as under the real selection (the same algorithmic FLOPs)."""
    nb = (w.S_k + w.block_size - 1) // w.block_size
    r = torch.arange(w.S_q, device=dev)
    qb = (w.S_k - w.S_q + r) // w.block_size
    j = torch.arange(nb, device=dev)
    cand = (j[None, :] >= w.n_init) & (j[None, :] <= (qb - w.n_local)[:, None])
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    heads = w.B * w.H_kv
    shared_key = torch.rand(heads, (w.S_q + 15) // 16, nb, device=dev, generator=g)[:, r // 16]
    own_key = torch.rand(heads, w.S_q, nb, device=dev, generator=g)
    n_sh = int(round(frac * w.topk))
    neg = torch.tensor(-1.0, device=dev)
    parts, taken = [], torch.zeros(heads, w.S_q, nb, dtype=torch.bool, device=dev)
    if n_sh:
        val, ix = torch.where(cand, shared_key, neg).topk(n_sh, dim=-1)
        taken.scatter_(-1, ix, val >= 0)
        parts.append(torch.where(val >= 0, ix, -1))
    if w.topk - n_sh:
        val, ix = torch.where(cand & ~taken, own_key, neg).topk(w.topk - n_sh, dim=-1)
        parts.append(torch.where(val >= 0, ix, -1))
    ix = torch.cat(parts, -1)
    ix = torch.where(ix < 0, nb + 1, ix).sort(dim=-1).values
    ix = torch.where(ix > nb, -1, ix).to(torch.int32)
    return ix.view(w.B, w.H_kv, w.S_q, w.topk).contiguous()


def event_ms(torch, f, n, warm=1, warm_s=0.1):
    """Average ms of n back-to-back calls of f (HIP events on the current
    stream), after at least `warm` calls and warm_s seconds of calls: the
    clocks drop while the host runs the oracle, and short kernels timed right
    after such a pause run up to about 1.6x slower."""
    t0 = time.perf_counter()
    i = 0
    while i < warm or time.perf_counter() - t0 < warm_s:
        f()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(n):
        f()
    c1.record()
    torch.cuda.synchronize()
    return c0.elapsed_time(c1) / n


def config_entry(w, torch, tb, workloads, dev, with_cpu, steps=10):
    """One prefill workload of the five: the whole step through the switch
    entry point (dense or compress -> select -> sparse), its stages, this
    build's dense attention at the same shape, and the oracle on a bounded
    sample of rows."""
    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    sparse_f, dense_f, select_f, _ = flop_counts(w)
    plan = tb.AttnPlan(w.B, w.H_q, w.H_kv, w.S_q, w.S_k, w.D, w.block_size, w.topk, w.n_init, w.n_local,
                       w.switch_len, None, dev)
    step_ms = event_ms(torch, lambda: plan.run(q, k, v), steps, warm=2)
    dense_ms = event_ms(torch, lambda: tb.dense_attn_fwd(q, k, v, causal=True), 3)
    e = {"path": "dense" if plan.dense else "sparse", "B": w.B, "S_q": w.S_q, "S_k": w.S_k, "H_q": w.H_q,
         "H_kv": w.H_kv, "topk": w.topk, "values": w.values, "step_ms": round(step_ms, 4),
         "dense_attn_ms": round(dense_ms, 4),
         "dense_attn_tflops": round(dense_f / (dense_ms * 1e-3) / 1e12, 2),
         "speedup_vs_dense": round(dense_ms / step_ms, 3)}
    if plan.dense:
        e["step_tflops"] = round(dense_f / (step_ms * 1e-3) / 1e12, 2)
        e["mfma_peak_frac"] = round(e["step_tflops"] / PEAK_BF16_TFLOPS, 4)
    else:
        kc = tb.compress_k(k)
        idx = tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local)
        attn_ms = event_ms(torch, lambda: tb.sparse_attn_fwd(q, k, v, idx, w.n_init, w.n_local), steps)
        sel_ms = event_ms(torch, lambda: tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local), steps)
        e.update({"sparse_attn_ms": round(attn_ms, 4), "select_ms": round(sel_ms, 4),
                  "compress_ms": round(event_ms(torch, lambda: tb.compress_k(k), steps), 4),
                  "step_tflops": round(sparse_f / (step_ms * 1e-3) / 1e12, 2),
                  "sparse_attn_tflops": round(sparse_f / (attn_ms * 1e-3) / 1e12, 2),
                  "mfma_peak_frac_attn": round(sparse_f / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "mfma_peak_frac_select": round(select_f / (sel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "algorithmic_flops": {"sparse_attn": sparse_f, "dense_attn": dense_f, "select": select_f}})
        del kc, idx
    if with_cpu:
        cb = cpu_baseline(w, x, target_s=4.0 if w.S_q <= 32768 else 6.0)
        e["cpu_baseline"] = {kk: cb[kk] for kk in ("unit", "cores", "kind", "sample")}
        e["cpu_baseline"]["value"] = round(cb["value"], 6)
        e["cpu_baseline"]["step_s_estimate"] = round(cb["step_s_estimate"], 3)
    del q, k, v, x, plan
    torch.cuda.empty_cache()
    return e


def decode_contiguous_entry(torch, tb, workloads, dev, with_cpu, reps=20):
    """The decode workload as stated (16 sequences, one query each, a
    contiguous 32768-key cache per sequence): a step is selection + sparse
    attention over compressed keys computed once beforehand (the compression
    of the whole cache is reported apart); against HBM, the step moves the
    attended K/V rows, the compressed keys and Q, O."""
    import numpy as np
    w = workloads.DECODE_32K
    x = workloads.make_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kc = tb.compress_k(k)
    idx = tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local)

    def step():
        i2 = tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local)
        tb.sparse_attn_fwd(q, k, v, i2, w.n_init, w.n_local)

    step_ms = event_ms(torch, step, reps, warm=2)
    attn_ms = event_ms(torch, lambda: tb.sparse_attn_fwd(q, k, v, idx, w.n_init, w.n_local), reps)
    sel_ms = event_ms(torch, lambda: tb.select_blocks(q, kc, w.S_k, w.topk, w.n_init, w.n_local), reps)
    comp_ms = event_ms(torch, lambda: tb.compress_k(k), 5)
    dense_ms = event_ms(torch, lambda: tb.dense_attn_fwd(q, k, v, causal=True), 5)
    per = w.topk + w.n_init + w.n_local
    kv = w.B * w.H_kv * min(per, w.S_k // 64) * 64 * w.D * 2 * 2
    kcb = w.B * w.H_kv * (w.S_k // 64) * w.D * 2
    qo = 2 * w.B * w.H_q * w.D * 2
    dense_bytes = w.B * w.H_kv * w.S_k * w.D * 2 * 2 + qo
    e = {"path": "sparse", "B": w.B, "S_q": w.S_q, "S_k": w.S_k, "H_q": w.H_q, "H_kv": w.H_kv, "topk": w.topk,
         "step_ms": round(step_ms, 4), "select_ms": round(sel_ms, 4), "sparse_attn_ms": round(attn_ms, 4),
         "compress_whole_cache_ms": round(comp_ms, 4), "dense_attn_ms": round(dense_ms, 4),
         "speedup_vs_dense": round(dense_ms / step_ms, 3),
         "hbm_roofline": {"step_bytes": kv + kcb + qo, "step_tbs": round((kv + kcb + qo) / (step_ms * 1e-3) / 1e12, 3),
                          "step_frac": round((kv + kcb + qo) / (step_ms * 1e-3) / 8e12, 4),
                          "attn_bytes": kv + qo, "attn_frac": round((kv + qo) / (attn_ms * 1e-3) / 8e12, 4),
                          "dense_bytes": dense_bytes,
                          "dense_frac": round(dense_bytes / (dense_ms * 1e-3) / 8e12, 4), "peak_tbs": 8.0}}
    if with_cpu:
        import oracle.infv2_oracle as O
        t0 = time.perf_counter()
        bs = [0, 5, 10, 15]
        k64, v64 = k[bs].double().cpu().numpy(), v[bs].double().cpu().numpy()
        q64 = q[bs].double().cpu().numpy()
        _, kco = O.compress_k(k64, 64)
        t1 = time.perf_counter()
        ix = O.select_blocks(q64, kco, w.S_k, w.topk, w.n_init, w.n_local, 64, 1 / math.sqrt(w.D))
        O.sparse_attn(q64, k64, v64, ix, 64, w.n_init, w.n_local, 1 / math.sqrt(w.D))
        t2 = time.perf_counter()
        e["cpu_baseline"] = {"kind": "oracle", "unit": "ms per step", "value": round((t2 - t1) / len(bs) * w.B * 1e3, 3),
                             "sample": (f"select + attend of {len(bs)} of the 16 sequences ({t2 - t1:.2f} s) scaled "
                                        f"to 16; their key compression took {t1 - t0:.2f} s apart"),
                             "cores": blas_threads()}
    del q, k, v, x, kc, idx
    torch.cuda.empty_cache()
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_prefill_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--profile-attn", type=int, default=0,
                    help="only launch the sparse attention kernel this many times (for counter runs)")
    ap.add_argument("--profile-bwd", type=int, default=0,
                    help="only run the sparse attention backward this many times (for profiler runs)")
    ap.add_argument("--profile-kernels", type=int, default=0,
                    help="for counter runs: launch each kernel family of the path this many times at the "
                         "workload's shape (compress, select, sparse attention, dense attention, backward, the "
                         "compressed branch alone and fused with the sparse attention) and the paged decode step "
                         "(attention, combine, selection, append), then exit")
    ap.add_argument("--no-bwd", action="store_true", help="skip timing the sparse attention backward")
    ap.add_argument("--no-decode", action="store_true", help="skip timing the paged decode step")
    ap.add_argument("--no-compressed", action="store_true",
                    help="skip timing the compressed-attention branch and the mixed output")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other four workloads (tiny 2k, 4k/8k switch, decode, 128k)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import trainable_block_sparse_mean_amd as tb
    import workloads

    wl = {w.name: w for w in workloads.ALL}[args.workload]
    wl = wl.with_(switch_len=0) if wl.S_k > wl.switch_len else wl
    dev = torch.device("cuda:0")
    x = workloads.make_inputs(wl)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    torch.cuda.synchronize()
    sparse_flops, dense_flops, select_flops, _ = flop_counts(wl)

    if args.profile_attn:
        kc = tb.compress_k(k)
        idx = tb.select_blocks(q, kc, wl.S_k, wl.topk, wl.n_init, wl.n_local)
        # a plain copy of known size, to calibrate the HBM byte counters
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        for _ in range(args.profile_attn):
            tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local)
        torch.cuda.synchronize()
        print(json.dumps({"profile_attn_launches": args.profile_attn, "copy_bytes": 2 * a.numel()}))
        return
    if args.profile_bwd:
        idx = tb.select_blocks(q, tb.compress_k(k), wl.S_k, wl.topk, wl.n_init, wl.n_local)
        o, lse = tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local)
        dout = seeded_dout(q, torch)
        # the same calibration copy as for --profile-attn
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(a).copy_(a)
        for _ in range(args.profile_bwd):
            tb.sparse_attn_bwd(q, k, v, o, lse, dout, idx, wl.n_init, wl.n_local)
        torch.cuda.synchronize()
        print(json.dumps({"profile_bwd_runs": args.profile_bwd}))
        return

    if args.profile_kernels:
        n = args.profile_kernels
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)   # calibration copy of known size
        torch.empty_like(a).copy_(a)
        for _ in range(n):
            kc = tb.compress_k(k)
        for _ in range(n):
            idx = tb.select_blocks(q, kc, wl.S_k, wl.topk, wl.n_init, wl.n_local)
        for _ in range(n):
            o, lse = tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local)
        for _ in range(n):
            tb.dense_attn_fwd(q, k, v, causal=True)
        dout = seeded_dout(q, torch)
        for _ in range(n):
            tb.sparse_attn_bwd(q, k, v, o, lse, dout, idx, wl.n_init, wl.n_local)
        vc = tb.compress_v(v)
        for _ in range(n):
            tb.compressed_attn_fwd(q, kc, vc, wl.S_k, return_lse=False)
        for _ in range(n):
            tb.mixed_attn_fwd(q, k, v, idx, kc, vc, 0.5, 0.5, wl.n_init, wl.n_local, return_lse=False)
        torch.cuda.synchronize()
        del o, lse, dout, idx, kc, vc
        time_decode_paged(torch, tb, workloads, dev, reps=n)
        torch.cuda.synchronize()
        print(json.dumps({"profile_kernels_launches": n, "copy_bytes": 2 * a.numel()}))
        return

    plan = tb.AttnPlan(wl.B, wl.H_q, wl.H_kv, wl.S_q, wl.S_k, wl.D, wl.block_size, wl.topk, wl.n_init,
                       wl.n_local, wl.switch_len, None, dev)
    for _ in range(args.warmup):
        plan.run(q, k, v)
    torch.cuda.synchronize()

    # ---- timed steps: the whole path, back to back -------------------------------
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        plan.run(q, k, v)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    ms_step = e0.elapsed_time(e1) / args.steps

    # ---- per stage, HIP events around each entry point (one kernel each) --------
    stages = {"compress": 0.0, "select": 0.0, "sparse_attn": 0.0}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    reps = max(3, args.steps)
    attn_calls = []
    for _ in range(reps):
        ev[0].record()
        kc = tb.compress_k(k)
        ev[1].record()
        idx = tb.select_blocks(q, kc, wl.S_k, wl.topk, wl.n_init, wl.n_local)
        ev[2].record()
        tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local)
        ev[3].record()
        torch.cuda.synchronize()
        stages["compress"] += ev[0].elapsed_time(ev[1]) / reps
        stages["select"] += ev[1].elapsed_time(ev[2]) / reps
        stages["sparse_attn"] += ev[2].elapsed_time(ev[3]) / reps
        attn_calls.append(ev[2].elapsed_time(ev[3]))

    # ---- the same call with a cold last-level cache: 512 MiB written between
    # calls (outside the timed events) evicts the 256 MB MALL, which otherwise
    # holds the whole K/V of one layer at 32k ---------------------------------
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold_calls = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        ev[0].record()
        tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local, return_lse=False)
        ev[1].record()
        torch.cuda.synchronize()
        cold_calls.append(ev[0].elapsed_time(ev[1]))
    del flush
    gemm_tflops = measured_gemm_tflops(torch, dev)

    dense_ms = None
    if not args.no_dense:
        tb.dense_attn_fwd(q, k, v, causal=True)
        torch.cuda.synchronize()
        dreps = 3
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for _ in range(dreps):
            tb.dense_attn_fwd(q, k, v, causal=True)
        d1.record()
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / dreps

    # ---- the backward of the sparse attention (training), same shape ------------
    bwd_ms = None
    if not args.no_bwd:
        idx = tb.select_blocks(q, tb.compress_k(k), wl.S_k, wl.topk, wl.n_init, wl.n_local)
        o, lse = tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local)
        dout = seeded_dout(q, torch)
        tb.sparse_attn_bwd(q, k, v, o, lse, dout, idx, wl.n_init, wl.n_local)
        torch.cuda.synchronize()
        breps = 3
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(breps):
            tb.sparse_attn_bwd(q, k, v, o, lse, dout, idx, wl.n_init, wl.n_local)
        b1.record()
        torch.cuda.synchronize()
        bwd_ms = b0.elapsed_time(b1) / breps
        del o, lse, dout

    decode = None if args.no_decode else time_decode_paged(torch, tb, workloads, dev)

    # ---- selection with the strided (approximate) LSE: time and recall ---------
    strided = {}
    kc = tb.compress_k(k)
    exact = tb.select_blocks(q, kc, wl.S_k, wl.topk, wl.n_init, wl.n_local)
    valid = exact >= 0
    for stride in (2, 4, 8):
        run = lambda: tb.select_blocks_strided_lse(q, kc, wl.S_k, wl.topk, stride, wl.n_init, wl.n_local)
        approx = run()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(5):
            run()
        s1.record()
        torch.cuda.synchronize()
        hit = (exact.unsqueeze(-1) == approx.unsqueeze(-2)).any(dim=-1) & valid
        strided[str(stride)] = {"select_ms": round(s0.elapsed_time(s1) / 5, 4),
                                "recall": round(float(hit.sum()) / max(float(valid.sum()), 1.0), 4)}
        del approx, hit
    del exact, valid

    # ---- the sparse kernel's dependence on how much a window's tokens share:
    # the same shape and FLOPs, with synthetic selections in which the 16
    # tokens of each window share 0, 1/2 or all of their top-k blocks --------
    shared = {}
    for frac in (0.0, 0.5, 1.0):
        sidx = shared_selection(torch, wl, frac, dev)
        ms = event_ms(torch, lambda: tb.sparse_attn_fwd(q, k, v, sidx, wl.n_init, wl.n_local, return_lse=False), 10)
        tf = sparse_flops / (ms * 1e-3) / 1e12
        shared[str(frac)] = {"sparse_attn_ms": round(ms, 4), "tflops": round(tf, 2),
                             "mfma_peak_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del sidx
    torch.cuda.empty_cache()

    # ---- the compressed-attention branch, alone and mixed with the sparse output --
    compressed = None
    if not args.no_compressed:
        # one (query head, visible compressed key) pair costs 4 D flops, as for
        # a key of the sparse attention: the same pairs and count as the two
        # scoring passes of selection (2 x 2 D each)
        cmp_flops = select_flops
        kc, vc = tb.compress_k(k), tb.compress_v(v)
        idx = tb.select_blocks(q, kc, wl.S_k, wl.topk, wl.n_init, wl.n_local)
        o_sp, _ = tb.sparse_attn_fwd(q, k, v, idx, wl.n_init, wl.n_local)
        buf = torch.empty_like(q)

        def mixed_step():
            kc2, vc2 = tb.compress_k(k), tb.compress_v(v)
            idx2 = tb.select_blocks(q, kc2, wl.S_k, wl.topk, wl.n_init, wl.n_local)
            o2, _ = tb.sparse_attn_fwd(q, k, v, idx2, wl.n_init, wl.n_local, return_lse=False)
            tb.compressed_attn_fwd(q, kc2, vc2, wl.S_k, o_sparse=o2, w_sparse=0.5, w_cmp=0.5, out=o2,
                                   return_lse=False)

        def fused_mixed_step():
            kc2, vc2 = tb.compress_k(k), tb.compress_v(v)
            idx2 = tb.select_blocks(q, kc2, wl.S_k, wl.topk, wl.n_init, wl.n_local)
            tb.mixed_attn_fwd(q, k, v, idx2, kc2, vc2, 0.5, 0.5, wl.n_init, wl.n_local, return_lse=False)

        def avg_ms(f, n=5):
            f()
            torch.cuda.synchronize()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            for _ in range(n):
                f()
            c1.record()
            torch.cuda.synchronize()
            return c0.elapsed_time(c1) / n

        branch_ms = avg_ms(lambda: tb.compressed_attn_fwd(q, kc, vc, wl.S_k, out=buf, return_lse=False))
        mix_ms = avg_ms(lambda: tb.compressed_attn_fwd(q, kc, vc, wl.S_k, o_sparse=o_sp, w_sparse=0.5, w_cmp=0.5,
                                                       out=buf, return_lse=False))
        compressed = {"branch_ms": round(branch_ms, 4),
                      "branch_tflops": round(cmp_flops / (branch_ms * 1e-3) / 1e12, 2),
                      "branch_mixed_ms": round(mix_ms, 4),
                      "compress_v_ms": round(avg_ms(lambda: tb.compress_v(v)), 4),
                      "mixed_step_ms": round(avg_ms(mixed_step), 4),
                      "fused_mixed_attn_ms": round(avg_ms(lambda: tb.mixed_attn_fwd(
                          q, k, v, idx, kc, vc, 0.5, 0.5, wl.n_init, wl.n_local, return_lse=False)), 4),
                      "fused_mixed_step_ms": round(avg_ms(fused_mixed_step), 4),
                      "branch_flops": cmp_flops}
        del kc, vc, idx, o_sp, buf

    # ---- the other workloads of the five, each measured the same way ---------------
    configs = None
    if not args.no_configs:
        del plan
        torch.cuda.empty_cache()
        configs = {}
        for w in (workloads.TINY, workloads.SWITCH_DENSE, workloads.SWITCH_SPARSE, workloads.EXTREME_128K):
            configs[w.name] = config_entry(w, torch, tb, workloads, dev, not args.no_cpu_baseline)
            print(f"[bench] {w.name}: {configs[w.name]['step_ms']} ms", file=sys.stderr, flush=True)
        configs[workloads.DECODE_32K.name] = decode_contiguous_entry(torch, tb, workloads, dev,
                                                                     not args.no_cpu_baseline)

    attn_tflops = sparse_flops / (stages["sparse_attn"] * 1e-3) / 1e12
    value = sparse_flops / (ms_step * 1e-3) / 1e12
    traffic = stored_traffic()
    roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, x)
        cpu = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample")}
        cpu["value"] = round(cpu["value"], 6)
        cpu["cpu_model"] = cpu_model()
        cpu["host_cpus"] = os.cpu_count()

    out = {
        "metric": "sparse-attn fwd ms & effective TFLOP/s at 32k; speedup vs dense; % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "S_q": wl.S_q, "S_k": wl.S_k, "H_q": wl.H_q,
                   "H_kv": wl.H_kv, "D": wl.D, "block_size": wl.block_size, "topk": wl.topk,
                   "n_init": wl.n_init, "n_local": wl.n_local, "values": wl.values,
                   "parallelism": "none (1 GPU)"},
        "stage_ms": {kk: round(vv, 4) for kk, vv in stages.items()},
        "sparse_attn_ms": round(stages["sparse_attn"], 4),
        "sparse_attn_tflops": round(attn_tflops, 2),
        "mfma_peak_frac_attn": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "mfma_peak_frac_step": round(value / PEAK_BF16_TFLOPS, 4),
        "sparse_attn_call_ms": dist(attn_calls),
        "sparse_attn_cold_mall_ms": dist(cold_calls),
        "measured_gemm_tflops": round(gemm_tflops, 1),
        "frac_of_measured_gemm": round(attn_tflops / gemm_tflops, 4),
        "dense_attn_ms": None if dense_ms is None else round(dense_ms, 4),
        "dense_attn_tflops": None if dense_ms is None else round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms_step, 3),
        "sparse_attn_bwd_ms": None if bwd_ms is None else round(bwd_ms, 4),
        "sparse_attn_bwd_tflops": None if bwd_ms is None else round(2 * sparse_flops / (bwd_ms * 1e-3) / 1e12, 2),
        "stage_mfma_frac": {
            "select": round(select_flops / (stages["select"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "sparse_attn": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "sparse_attn_bwd": None if bwd_ms is None else
            round(2 * sparse_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "dense_attn": None if dense_ms is None else
            round(dense_flops / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "decode_b16_32k_paged": decode,
        "select_strided_lse": strided,
        "sparse_attn_shared_selection": shared,
        "compressed_branch": compressed,
        "configs": configs,
        "algorithmic_flops": {"sparse_attn": sparse_flops, "dense_attn": dense_flops, "select": select_flops,
                              "sparse_attn_bwd": 2 * sparse_flops},
        "wall_ms_per_step": round(wall_ms, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
