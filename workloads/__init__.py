"""Seeded synthetic attention workloads.

This module only describes shapes and draws random inputs.  It holds none of
the attention arithmetic, so both the fp64 oracle's tests and the GPU path's
tests and benchmark can use it without sharing any of the method's code.

The five workloads are the pages' own examples of FlashAttention-2 regimes:
  * fp32_small    -- a tiny fp32 correctness case;
  * short_seq     -- many short sequences (the explainer's Legacy section notes
                     gains shrink there; bandwidth-leaning);
  * mid_seq       -- a mid-length, non-causal case;
  * long_causal   -- 2 sequences x 16 heads x 8192 tokens, Saraf §2.3's
                     example, causal, with 0.1% of Q and K entries scaled x20
                     so the running max has to be corrected;
  * long_few_head -- 1 x 2 heads x 32768 tokens, the explainer's
                     "few heads, long sequence" occupancy case.

Recipe (the same for every workload):
  1. one CPU ``torch.Generator`` seeded with ``seed``;
  2. Q, K, V drawn in that order as float32 N(0, 1), shape [B, H, N, d];
  3. if ``outlier_frac`` > 0: independent Bernoulli(outlier_frac) masks for
     Q then K (from the same generator, uniform < frac); masked entries are
     multiplied by ``outlier_mult`` in float32 (V untouched);
  4. cast to the workload dtype (bf16 uses round-to-nearest-even).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "HEADLINE", "make_inputs", "make_grad_output", "credited_flops",
           "credited_bwd_flops", "credited_pairs", "get"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "fp32" or "bf16"
    scale: float
    causal: bool
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "B": self.B, "H": self.H, "N": self.N, "d": self.d,
            "dtype": self.dtype, "causal": self.causal, "scale": self.scale,
            "outlier_frac": self.outlier_frac, "outlier_mult": self.outlier_mult,
        }


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp32_small", 1, 1, 128, 64, "fp32", 1.0 / math.sqrt(64), False),
        Workload("short_seq", 32, 16, 512, 64, "bf16", 1.0 / 8.0, False),
        Workload("mid_seq", 8, 16, 2048, 128, "bf16", 1.0 / math.sqrt(128), False),
        Workload("long_causal", 2, 16, 8192, 128, "bf16", 1.0 / math.sqrt(128), True, 0.001, 20.0),
        Workload("long_few_head", 1, 2, 32768, 128, "bf16", 1.0 / math.sqrt(128), True),
    ]
}

# The workload the headline throughput is quoted on (d=128, N=8192, causal).
HEADLINE = "long_causal"


def get(name: str) -> Workload:
    return WORKLOADS[name]


def make_inputs(w: Workload, seed: int, device="cpu"):
    """Draw (q, k, v) for workload ``w`` with ``seed``; returns tensors on ``device``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = w.shape
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.outlier_frac > 0.0:
        mq = torch.rand(shape, generator=g) < w.outlier_frac
        mk = torch.rand(shape, generator=g) < w.outlier_frac
        q = torch.where(mq, q * w.outlier_mult, q)
        k = torch.where(mk, k * w.outlier_mult, k)
    dt = w.torch_dtype
    return (q.to(dt).to(device), k.to(dt).to(device), v.to(dt).to(device))


def make_grad_output(w: Workload, seed: int, device="cpu"):
    """Draw the upstream gradient dO for workload ``w``: float32 N(0, 1) of
    shape [B, H, N, d] from a CPU generator seeded with ``seed`` (use a seed
    distinct from the one the inputs were drawn with), cast to the workload
    dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(w.shape, generator=g, dtype=torch.float32).to(w.torch_dtype).to(device)


def credited_bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Credited attention-backward work: the four N x N x d products
    (S, dP, dV, and one of dQ / dK) plus the fifth, 10*B*H*N^2*d in all,
    halved when causal."""
    f = 10.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def credited_pairs(N: int, window_left: int, window_right: int) -> int:
    """Number of (query, key) pairs of one head that a sliding window
    (-1 = unbounded side) leaves visible: sum over queries i of the keys j
    with max(0, i - wl) <= j <= min(N - 1, i + wr).  (-1, 0) gives the
    causal N(N+1)/2, (-1, -1) gives N^2."""
    i = torch.arange(N, dtype=torch.int64)
    lo = torch.clamp(i - window_left, min=0) if window_left >= 0 else torch.zeros_like(i)
    hi = torch.clamp(i + window_right, max=N - 1) if window_right >= 0 else torch.full_like(i, N - 1)
    return int((hi - lo + 1).clamp(min=0).sum())


def credited_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Credited attention-forward work: 4*B*H*N^2*d, halved when causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def make_block_mask(n_layouts: int, n_qblocks: int, n_kblocks: int, density: float, seed: int,
                    keep_diagonal: bool = True):
    """Seeded random block-sparse pattern, bool [n_layouts, n_qblocks,
    n_kblocks]: each block set with probability ``density`` (a CPU
    torch.Generator seeded with ``seed``), plus the diagonal blocks when
    ``keep_diagonal`` (so that, with square blocks, every query sees a key)."""
    g = torch.Generator().manual_seed(seed)
    m = torch.rand((n_layouts, n_qblocks, n_kblocks), generator=g) < density
    if keep_diagonal:
        idx = torch.arange(min(n_qblocks, n_kblocks))
        m[:, idx, idx] = True
    return m.numpy()


def credited_pairs_block_sparse(N: int, block_mask, block_q: int, block_k: int, causal: bool) -> int:
    """Visible (query, key) pairs of one layout: for every set block, the
    pairs of its (ragged) row and key ranges, only those with j <= i when
    causal."""
    import numpy as np

    bm = np.asarray(block_mask).astype(bool)
    total = 0
    for qb, kb in zip(*np.nonzero(bm)):
        r0, r1 = qb * block_q, min(N, (qb + 1) * block_q)
        c0, c1 = kb * block_k, min(N, (kb + 1) * block_k)
        if not causal:
            total += (r1 - r0) * (c1 - c0)
            continue
        i = np.arange(r0, r1)
        total += int(np.clip(np.minimum(i, c1 - 1) - c0 + 1, 0, None).sum())
    return int(total)


def make_paged_cache(context_lens, H_kv: int, d: int, page_size: int, seed: int, spare_pages: int = 3,
                     device="cpu"):
    """Seeded paged key/value cache for decoding: caches [n_pages, page_size,
    H_kv, d] bf16 filled with randn (unused slots too), and an int32 page
    table [B, max_pages] assigning each sequence's logical pages to randomly
    permuted physical pages (entries past a sequence's pages are -1).
    Returns (k_cache, v_cache, page_table)."""
    g = torch.Generator().manual_seed(seed)
    need = [-(-int(L) // page_size) for L in context_lens]
    n_pages = sum(need) + spare_pages
    max_pages = max(max(need), 1)
    k = torch.randn((n_pages, page_size, H_kv, d), generator=g).to(torch.bfloat16)
    v = torch.randn((n_pages, page_size, H_kv, d), generator=g).to(torch.bfloat16)
    perm = torch.randperm(n_pages, generator=g)
    table = torch.full((len(context_lens), max_pages), -1, dtype=torch.int32)
    nxt = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[nxt:nxt + n].to(torch.int32)
        nxt += n
    return k.to(device), v.to(device), table.to(device)


def make_signs(d: int, seed: int):
    """Seeded random +-1 vector of length d (float32 numpy array), the
    signs of the FP8 rotation."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (d,), generator=g) * 2 - 1).to(torch.float32).numpy()
