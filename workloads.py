"""Seeded synthetic inputs for the InfLLM-V2 block-sparse attention path.

This module only draws random numbers and arranges them into tensors of the
shapes the workloads use.  It holds none of the method's arithmetic (no block
means, no scores, no selection, no attention): both the fp64 oracle and the
HIP path receive the very same tensors from here.

Layout of every tensor is [B, H, S, D] contiguous, bf16, following the shape
docstrings of the sparse-pattern functions on the skill page "Infllm V2 Dense
Sparse Switchable Attention" (Step 2: Sparse Pattern Selection Module).

Each generator returns a dict with ``q``, ``k``, ``v`` (torch bf16 tensors on
the CPU) and the parameters of the workload.  Values are drawn in fp32 from a
``torch.Generator`` seeded with ``seed`` and rounded to bf16 (round to nearest
even) by torch.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    S_q: int
    S_k: int
    D: int = 128
    block_size: int = 64
    topk: int = 64
    n_init: int = 1
    n_local: int = 2
    switch_len: int = 0          # dense iff S_k <= switch_len
    values: str = "normal"       # recipe name, see make_inputs
    seed: int = 0

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Sizes, block size, top-k, initial/sliding block counts
# and value recipes are those of the long-context workload list this library
# is measured on; the page itself prints no shapes.
TINY = Workload("tiny_prefill_2k", B=1, H_q=8, H_kv=1, S_q=2048, S_k=2048,
                topk=8, n_init=1, n_local=2, switch_len=0, values="normal")
TINY_PRESCALED = TINY.with_(name="tiny_prefill_2k_prescaled", values="prescaled")
SWITCH_DENSE = Workload("switch_4k_dense", B=1, H_q=32, H_kv=2, S_q=4096, S_k=4096,
                        topk=16, switch_len=4096, values="planted")
SWITCH_SPARSE = SWITCH_DENSE.with_(name="switch_8k_sparse", S_q=8192, S_k=8192)
LONG_32K = Workload("long_prefill_32k", B=1, H_q=32, H_kv=2, S_q=32768, S_k=32768,
                    topk=64, switch_len=0, values="normal")
DECODE_32K = Workload("decode_b16_32k", B=16, H_q=32, H_kv=2, S_q=1, S_k=32768,
                      topk=64, switch_len=0, values="normal")
EXTREME_128K = Workload("extreme_prefill_128k", B=1, H_q=32, H_kv=2, S_q=131072,
                        S_k=131072, topk=128, switch_len=0, values="clustered")

ALL = [TINY, SWITCH_DENSE, SWITCH_SPARSE, LONG_32K, DECODE_32K, EXTREME_128K]


def _randn(gen: torch.Generator, *shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def make_inputs(w: Workload) -> dict:
    """Draw q, k, v for workload ``w`` (CPU bf16, [B,H,S,D])."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    if w.values == "normal":
        q = _randn(gen, w.B, w.H_q, w.S_q, w.D)
        k = _randn(gen, w.B, w.H_kv, w.S_k, w.D)
        v = _randn(gen, w.B, w.H_kv, w.S_k, w.D)
    elif w.values == "prescaled":
        # literal reading of "N(0,1) scaled by 1/sqrt(head_dim)"
        s = 1.0 / math.sqrt(w.D)
        q = _randn(gen, w.B, w.H_q, w.S_q, w.D) * s
        k = _randn(gen, w.B, w.H_kv, w.S_k, w.D) * s
        v = _randn(gen, w.B, w.H_kv, w.S_k, w.D) * s
    elif w.values == "planted":
        q, k, v = _planted(gen, w)
    elif w.values == "clustered":
        q, k, v = _clustered(gen, w)
    elif w.values == "constant_k":
        # every key identical: every block score ties
        q = _randn(gen, w.B, w.H_q, w.S_q, w.D)
        k = _randn(gen, w.B, w.H_kv, 1, w.D).expand(w.B, w.H_kv, w.S_k, w.D).contiguous()
        v = _randn(gen, w.B, w.H_kv, w.S_k, w.D)
    elif w.values == "integer":
        # small integers: every sum in a block mean is exact in any order
        q = torch.randint(-4, 5, (w.B, w.H_q, w.S_q, w.D), generator=gen).float()
        k = torch.randint(-8, 9, (w.B, w.H_kv, w.S_k, w.D), generator=gen).float()
        v = torch.randint(-2, 3, (w.B, w.H_kv, w.S_k, w.D), generator=gen).float()
    else:
        raise ValueError(f"unknown value recipe {w.values!r}")
    return dict(q=q.to(torch.bfloat16).contiguous(),
                k=k.to(torch.bfloat16).contiguous(),
                v=v.to(torch.bfloat16).contiguous())


def _planted(gen: torch.Generator, w: Workload):
    """One planted high-similarity key block per 64-token query chunk.

    For each query chunk c that has candidate blocks, draw a direction u_c and
    a target block p(c), uniform over the chunk's candidates
    [n_init, c - n_local].  Queries of chunk c (all heads) become
    (n + u_c)/sqrt(2); every key of block b becomes
    (n' + sum_{c: p(c)=b} u_c) / sqrt(1 + m_b), m_b = number of chunks
    planting b.  Returns (q, k, v) in fp32 and the plan via ``planted_targets``.
    """
    BS = w.block_size
    q = _randn(gen, w.B, w.H_q, w.S_q, w.D)
    k = _randn(gen, w.B, w.H_kv, w.S_k, w.D)
    v = _randn(gen, w.B, w.H_kv, w.S_k, w.D)
    off = w.S_k - w.S_q
    targets = planted_targets(w)
    n_chunks = (w.S_k + BS - 1) // BS
    add = torch.zeros(w.B, w.H_kv, n_chunks, w.D)
    cnt = torch.zeros(w.B, w.H_kv, n_chunks)
    for (b, g, c), p in targets.items():
        u = _randn(gen, w.D)
        r0 = max(c * BS - off, 0)
        r1 = min((c + 1) * BS - off, w.S_q)
        h0, h1 = g * w.G, (g + 1) * w.G
        q[b, h0:h1, r0:r1, :] = (q[b, h0:h1, r0:r1, :] + u) / math.sqrt(2.0)
        add[b, g, p] += u
        cnt[b, g, p] += 1
    for b in range(w.B):
        for g in range(w.H_kv):
            for p in torch.nonzero(cnt[b, g]).flatten().tolist():
                t0, t1 = p * BS, min((p + 1) * BS, w.S_k)
                k[b, g, t0:t1, :] = (k[b, g, t0:t1, :] + add[b, g, p]) / math.sqrt(1.0 + cnt[b, g, p])
    return q, k, v


def planted_targets(w: Workload) -> dict:
    """{(b, g, query_chunk): planted block} for the planted recipe (seeded)."""
    BS = w.block_size
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 1)
    off = w.S_k - w.S_q
    first_chunk = off // BS
    last_chunk = (w.S_k - 1) // BS
    out = {}
    for b in range(w.B):
        for g in range(w.H_kv):
            for c in range(first_chunk, last_chunk + 1):
                lo, hi = w.n_init, c - w.n_local
                if hi < lo:
                    continue
                out[(b, g, c)] = lo + int(torch.randint(0, hi - lo + 1, (1,), generator=gen))
    return out


def _clustered(gen: torch.Generator, w: Workload):
    """Keys from a mixture of 8 Gaussian clusters, chosen per 64-key block;
    queries biased toward clusters 0 and 1, so selection is skewed."""
    BS = w.block_size
    n_clusters = 8
    mu = _randn(gen, n_clusters, w.D)
    nb = (w.S_k + BS - 1) // BS
    z = torch.randint(0, n_clusters, (w.B, w.H_kv, nb), generator=gen)
    k = _randn(gen, w.B, w.H_kv, w.S_k, w.D)
    for b in range(w.B):
        for g in range(w.H_kv):
            centre = mu[z[b, g]].repeat_interleave(BS, dim=0)[: w.S_k]
            k[b, g] = (centre + k[b, g]) / math.sqrt(2.0)
    v = _randn(gen, w.B, w.H_kv, w.S_k, w.D)
    bias = 0.5 * (mu[0] + mu[1]) * math.sqrt(2.0)
    q = (_randn(gen, w.B, w.H_q, w.S_q, w.D) + bias) / math.sqrt(2.0)
    return q, k, v


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a bf16 tensor as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")
