"""Plain, slow fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code, tables or helpers
with the HIP kernels and imports nothing from the library package.

What it computes (the plain definition, written out):

    S_ij   = scale * sum_k q_ik * k_jk                  (full score rows)
    A_ij   = True if non-causal, else (j <= i)          (causal mask)
    m_i    = max_{j: A_ij} S_ij
    P_ij   = exp(S_ij - m_i) if A_ij else 0
    l_i    = sum_j P_ij
    O_i    = (sum_j P_ij * v_j) / l_i
    LSE_i  = m_i + ln(l_i)

Sources (web pages on FlashAttention-2):
  * Saraf, "FlashAttention 2: Three Places the Chip Was Still Waiting",
    section 1 (the naive kernel builds the full token-by-token score matrix;
    online softmax carries a running max and denominator and gives the exact
    answer) and section 3 (the tiled kernel's output is identical to standard
    attention; only the schedule changes).
  * papermap "FlashAttention-2" explainer, Chapter 02, "What stays true from
    FA1" (exact attention, identical outputs; the N x N matrix never reaches
    HBM in the fast kernel).
  * Mishra, "FlashAttention-2 and -3: From Algebra to GPU Scheduling",
    "Keep the unchanged mathematical target in view" (running max,
    denominator and numerator define the output; their merge identity is what
    makes tiling correct) and "Another use of mergeable statistics".

Readings where the pages are silent (each listed in the design notes):
  * the scale multiplies the raw dot products before the softmax;
  * causal means key j is visible to query i iff j <= i (equal lengths);
  * LSE is the natural log of sum_j exp(S_ij) over visible keys.

Everything here is float64 numpy.  Inputs of any float dtype are upcast
exactly (bf16 and fp32 values are exactly representable in fp64).

The module also holds the fp64 rendering of the pages' tiled algorithm
(``tiled_online_attention``), which walks key blocks with a running max and
denominator in the order the pages describe.  It is not the oracle; tests use
it to check the pages' exactness claims against the oracle.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "scores",
    "visible",
    "softmax_stats",
    "finalize",
    "attention_head",
    "attention_ref",
    "attention_rows",
    "probabilities",
    "partial_stats",
    "merge_stats",
    "tiled_online_attention",
    "kv_head_of",
    "attention_ref_gqa",
    "visible_window",
    "attention_head_window",
    "attention_ref_window",
    "probabilities_window",
    "visible_block_sparse",
    "layout_index",
    "attention_head_block_sparse",
    "attention_ref_block_sparse",
    "gather_pages",
    "visible_decode",
    "decode_paged_ref",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --- the definition, one step per function ---------------------------------

def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head: q [nq, d], k [nk, d] -> [nq, nk].

    Saraf §1: each score compares one query row with one key row.
    """
    return float(scale) * (q @ k.T)


def visible(row_ids, key_ids, causal: bool) -> np.ndarray:
    """Boolean mask [len(row_ids), len(key_ids)]; True where query row i may
    attend to key j.

    Causal reading: key j is visible to query i iff j <= i.
    """
    rows = np.asarray(row_ids)[:, None]
    cols = np.asarray(key_ids)[None, :]
    if not causal:
        return np.ones((rows.shape[0], cols.shape[1]), dtype=bool)
    return cols <= rows


def softmax_stats(s: np.ndarray, mask: np.ndarray, v: np.ndarray):
    """Row statistics over the visible keys of a score block.

    Returns (m, l, num): the row max of visible scores, the denominator
    sum exp(S - m) and the unnormalised numerator sum exp(S - m) v_j
    (Mishra, "Keep the unchanged mathematical target in view").
    Rows with no visible key get m = -inf, l = 0, num = 0.
    """
    s_vis = np.where(mask, s, -np.inf)
    m = s_vis.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    shift = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(np.where(mask, s - shift[:, None], -np.inf))
    l = p.sum(axis=1)
    num = p @ v
    return m, l, num


def finalize(m: np.ndarray, l: np.ndarray, num: np.ndarray):
    """O = num / l and LSE = m + ln l: the single normalisation at the end."""
    o = num / l[:, None]
    lse = m + np.log(l)
    return o, lse


def attention_head(q, k, v, scale: float, causal: bool, rows=None, row_block: int = 1024):
    """Exact attention for one head.

    q, k, v: [N, d] (upcast to fp64).  ``rows`` selects query rows (default:
    all).  Full score rows are materialised, ``row_block`` query rows at a
    time; nothing is tiled along the keys.
    Returns (O [len(rows), d], LSE [len(rows)]) in fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    row_ids = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((len(row_ids), v.shape[1]), dtype=np.float64)
    lse = np.empty(len(row_ids), dtype=np.float64)
    for start in range(0, len(row_ids), row_block):
        ids = row_ids[start:start + row_block]
        s = scores(q[ids], k, scale)
        mask = visible(ids, np.arange(k.shape[0]), causal)
        m, l, num = softmax_stats(s, mask, v)
        o[start:start + len(ids)], lse[start:start + len(ids)] = finalize(m, l, num)
    return o, lse


def attention_ref(q, k, v, scale: float, causal: bool, row_block: int = 1024):
    """Exact attention over [..., N, d] tensors (e.g. [B, H, N, d]).

    Returns (O [..., N, d], LSE [..., N]) as fp64 numpy arrays.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    n, dv = q.shape[-2], v.shape[-1]
    o = np.empty(lead + (n, dv), dtype=np.float64)
    lse = np.empty(lead + (n,), dtype=np.float64)
    for idx in np.ndindex(*lead):
        o[idx], lse[idx] = attention_head(q[idx], k[idx], v[idx], scale, causal, row_block=row_block)
    return o, lse


def attention_rows(q, k, v, scale: float, causal: bool, rows):
    """Exact attention for selected query rows of one head (sampled checks)."""
    return attention_head(q, k, v, scale, causal, rows=rows)


def probabilities(q, k, scale: float, causal: bool) -> np.ndarray:
    """Normalised attention probabilities P / l for one head, [N, N]."""
    q, k = _f64(q), _f64(k)
    ids = np.arange(q.shape[0])
    s = scores(q, k, scale)
    mask = visible(ids, np.arange(k.shape[0]), causal)
    s_vis = np.where(mask, s, -np.inf)
    m = s_vis.max(axis=1)
    p = np.exp(np.where(mask, s - m[:, None], -np.inf))
    return p / p.sum(axis=1, keepdims=True)


# --- mergeable statistics ---------------------------------------------------

def partial_stats(q, k, v, scale: float, causal: bool, key_ids):
    """(m, l, num) of every query row of one head over a subset of the keys.

    Mishra, "Keep the unchanged mathematical target in view" and "Another use
    of mergeable statistics": statistics of disjoint key sets can be combined
    exactly.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    key_ids = np.asarray(key_ids, dtype=np.int64)
    ids = np.arange(q.shape[0])
    s = scores(q, k[key_ids], scale)
    mask = visible(ids, key_ids, causal)
    return softmax_stats(s, mask, v[key_ids])


def merge_stats(parts):
    """Combine (m, l, num) of disjoint key sets into the statistics of their union.

    m = max_a m_a; each part is brought onto the common max by exp(m_a - m)
    before its denominator and numerator are added.
    """
    ms = np.stack([p[0] for p in parts])
    m = ms.max(axis=0)
    shift = np.where(np.isfinite(m), m, 0.0)
    l = np.zeros_like(parts[0][1])
    num = np.zeros_like(parts[0][2])
    for pm, pl, pnum in parts:
        w = np.where(np.isfinite(pm), np.exp(np.where(np.isfinite(pm), pm, 0.0) - shift), 0.0)
        l = l + w * pl
        num = num + w[:, None] * pnum
    return m, l, num


# --- the pages' tiled schedule, in fp64 (for checking the exactness claims) --

def tiled_online_attention(q, k, v, scale: float, causal: bool, block_rows: int = 64,
                           block_cols: int = 64, normalize_each_step: bool = False):
    """The tiled online-softmax algorithm of the pages, in fp64, for one head.

    Query rows are taken ``block_rows`` at a time (Saraf §2.3: independent
    query blocks).  Each block streams the key/value blocks past itself,
    keeping a running max m, denominator l and accumulator acc per row
    (Saraf §1).  When the running max rises, the banked terms are corrected
    by exp(m_old - m_new) (Saraf §2.2, the correction that cannot wait).

    normalize_each_step=False: acc stays unnormalised and is divided by l once
    per query block (the FlashAttention-2 schedule, Saraf §2.2).
    normalize_each_step=True: acc always holds the normalised output and is
    rescaled by l_old / l_new every step (the FlashAttention-1 schedule the
    same section describes).

    Returns (O [N, d], LSE [N], normalisations) where ``normalisations`` counts
    how often an accumulator block was divided.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, nk = q.shape[0], k.shape[0]
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    normalisations = 0
    for r0 in range(0, n, block_rows):
        ids = np.arange(r0, min(r0 + block_rows, n))
        m = np.full(len(ids), -np.inf)
        l = np.zeros(len(ids))
        acc = np.zeros((len(ids), v.shape[1]))
        for c0 in range(0, nk, block_cols):
            kids = np.arange(c0, min(c0 + block_cols, nk))
            mask = visible(ids, kids, causal)
            if not mask.any():
                continue
            s = scores(q[ids], k[kids], scale)
            s_vis = np.where(mask, s, -np.inf)
            m_new = np.maximum(m, s_vis.max(axis=1))
            shift = np.where(np.isfinite(m_new), m_new, 0.0)
            corr = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - shift), 0.0)
            p = np.exp(np.where(mask, s - shift[:, None], -np.inf))
            l_new = corr * l + p.sum(axis=1)
            if normalize_each_step:
                # acc holds O normalised by l; bring it to the new max and the
                # new denominator, then add this block's normalised share.
                keep = np.where(l_new > 0, corr * l / np.where(l_new > 0, l_new, 1.0), 0.0)
                acc = keep[:, None] * acc + (p @ v[kids]) / np.where(l_new > 0, l_new, 1.0)[:, None]
                normalisations += 1
            else:
                acc = corr[:, None] * acc + p @ v[kids]
            m, l = m_new, l_new
        if normalize_each_step:
            o[ids] = acc
        else:
            o[ids] = acc / l[:, None]
            normalisations += 1
        lse[ids] = m + np.log(l)
    return o, lse, normalisations


# --- grouped key/value heads (GQA / MQA) ------------------------------------

def kv_head_of(h: int, n_heads: int, n_kv_heads: int) -> int:
    """The key/value head query head ``h`` reads when ``n_heads`` query heads
    share ``n_kv_heads`` key/value heads in equal, consecutive groups."""
    return h // (n_heads // n_kv_heads)


def attention_ref_gqa(q, k, v, scale: float, causal: bool, row_block: int = 1024):
    """Exact attention with grouped key/value heads: q [B, H, N, d], k and v
    [B, H_kv, N, d] with H a multiple of H_kv; query head h attends with key
    and value head ``kv_head_of(h, H, H_kv)``.  Returns (O [B, H, N, d],
    LSE [B, H, N]) in fp64.

    papermap "FlashAttention-2" explainer, Chapter 03 ("The Downstream
    Story") and Chapter 05 ("The variant family"): GQA-aware kernels are
    among the variants built on the same partitioning; the grouping itself
    is the plain reading of the name.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, _ = q.shape
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError(f"{H} query heads cannot share {Hkv} key/value heads evenly")
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, g], v[b, g], scale, causal, row_block=row_block)
    return o, lse


# --- sliding-window (local) attention ---------------------------------------

def visible_window(row_ids, key_ids, window_left: int, window_right: int) -> np.ndarray:
    """Boolean mask [len(row_ids), len(key_ids)]: key j is visible to query i
    iff i - window_left <= j <= i + window_right, a negative bound meaning
    no limit on that side.  (-1, 0) is the causal mask, (-1, -1) none.

    papermap "FlashAttention-2" explainer, Chapter 03 ("The Downstream
    Story") and Chapter 05 ("The variant family") name sliding-window
    attention among the variants built on FlashAttention-2's partitioning;
    a band of keys around each query, bounded on either side, is the plain
    reading of the name.
    """
    rows = np.asarray(row_ids)[:, None]
    cols = np.asarray(key_ids)[None, :]
    vis = np.ones((rows.shape[0], cols.shape[1]), dtype=bool)
    if window_left >= 0:
        vis &= cols >= rows - window_left
    if window_right >= 0:
        vis &= cols <= rows + window_right
    return vis


def attention_head_window(q, k, v, scale: float, window_left: int, window_right: int):
    """Exact attention of one head under a sliding-window mask; every row
    must see at least one key (true whenever both bounds are >= 0 or
    unbounded).  Returns (O [N, d], LSE [N]) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    ids = np.arange(q.shape[0])
    s = scores(q, k, scale)
    mask = visible_window(ids, np.arange(k.shape[0]), window_left, window_right)
    m, l, num = softmax_stats(s, mask, v)
    return finalize(m, l, num)


def attention_ref_window(q, k, v, scale: float, window_left: int, window_right: int):
    """Sliding-window attention over [B, H, N, d] (k, v may have fewer heads:
    grouped heads as in ``attention_ref_gqa``).  Returns (O, LSE) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            o[b, h], lse[b, h] = attention_head_window(q[b, h], k[b, g], v[b, g], scale, window_left, window_right)
    return o, lse


def probabilities_window(q, k, scale: float, window_left: int, window_right: int) -> np.ndarray:
    """Normalised attention probabilities of one head under a sliding window."""
    q, k = _f64(q), _f64(k)
    ids = np.arange(q.shape[0])
    s = scores(q, k, scale)
    mask = visible_window(ids, np.arange(k.shape[0]), window_left, window_right)
    s_vis = np.where(mask, s, -np.inf)
    m = s_vis.max(axis=1)
    p = np.exp(np.where(mask, s - m[:, None], -np.inf))
    return p / p.sum(axis=1, keepdims=True)


# --- block-sparse masks ----------------------------------------------------------

def visible_block_sparse(row_ids, key_ids, block_mask, block_q: int, block_k: int, causal: bool) -> np.ndarray:
    """Boolean mask [len(row_ids), len(key_ids)] of a block-sparse pattern:
    key j is visible to query i iff block_mask[i // block_q, j // block_k]
    is set, and also j <= i when causal.

    papermap "FlashAttention-2" explainer, Chapter 03 ("The Downstream
    Story") and Chapter 05 ("The variant family") name block-sparse
    attention among the variants built on FlashAttention-2's partitioning;
    a mask given per (query block, key block) pair, the block sizes fixed,
    is the plain reading of the name.
    """
    rows = np.asarray(row_ids)
    cols = np.asarray(key_ids)
    bm = np.asarray(block_mask).astype(bool)
    vis = bm[(rows // block_q)[:, None], (cols // block_k)[None, :]]
    if causal:
        vis = vis & (cols[None, :] <= rows[:, None])
    return vis


def layout_index(b: int, h: int, n_batch: int, n_heads: int, n_layouts: int) -> int:
    """Which block mask (query) head h of sequence b uses: one mask for all
    (n_layouts = 1), one per head (n_layouts = H) or one per sequence and
    head (n_layouts = B*H, index b*H + h)."""
    if n_layouts == 1:
        return 0
    if n_layouts == n_heads:
        return h
    if n_layouts == n_batch * n_heads:
        return b * n_heads + h
    raise ValueError(f"{n_layouts} block masks fit neither 1, H={n_heads} nor B*H={n_batch * n_heads}")


def attention_head_block_sparse(q, k, v, scale: float, block_mask, block_q: int, block_k: int, causal: bool):
    """Exact attention of one head under a block-sparse mask.  A row that
    sees no key at all has no softmax; it gets O = 0 and LSE = -inf (the
    empty sum: exp(LSE) = 0).  Returns (O [N, d], LSE [N]) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    s = scores(q, k, scale)
    mask = visible_block_sparse(np.arange(n), np.arange(k.shape[0]), block_mask, block_q, block_k, causal)
    m, l, num = softmax_stats(s, mask, v)
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf)
    seen = l > 0
    if seen.any():
        o[seen], lse[seen] = finalize(m[seen], l[seen], num[seen])
    return o, lse


def attention_ref_block_sparse(q, k, v, scale: float, layouts, block_q: int, block_k: int, causal: bool):
    """Block-sparse attention over [B, H, N, d] (k, v may have fewer heads:
    grouped heads as in ``attention_ref_gqa``); ``layouts`` is [L, ceil(N /
    block_q), ceil(N / block_k)] with L chosen as in ``layout_index``.
    Returns (O, LSE) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    layouts = np.asarray(layouts)
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            mask = layouts[layout_index(b, h, B, H, layouts.shape[0])]
            o[b, h], lse[b, h] = attention_head_block_sparse(q[b, h], k[b, g], v[b, g], scale, mask,
                                                             block_q, block_k, causal)
    return o, lse



# --- decoding from a paged key/value cache -----------------------------------------

def gather_pages(cache, block_table_row, context_len: int, kv_head: int) -> np.ndarray:
    """The first ``context_len`` keys (or values) of one sequence and one
    key/value head, from a paged cache [n_pages, page_size, H_kv, d]:
    logical key j lives in physical page block_table_row[j // page_size] at
    slot j % page_size."""
    cache = np.asarray(cache)
    page_size = cache.shape[1]
    out = np.empty((context_len, cache.shape[3]), dtype=np.float64)
    for j in range(context_len):
        out[j] = cache[int(block_table_row[j // page_size]), j % page_size, kv_head]
    return out


def visible_decode(n_new: int, context_len: int) -> np.ndarray:
    """Boolean mask [n_new, context_len] for the n_new newest tokens of a
    sequence whose cache holds context_len keys (the new tokens' own keys
    included, last): new token i sits at position context_len - n_new + i
    and sees the keys at positions up to its own (the causal mask)."""
    pos = context_len - n_new + np.arange(n_new)
    return np.arange(context_len)[None, :] <= pos[:, None]


def decode_paged_ref(q, k_cache, v_cache, block_table, context_lens, scale: float):
    """Attention of the newest n_q tokens of each sequence over its paged
    cache.  q [B, H, n_q, d] (query heads grouped on the cache's H_kv heads
    as in ``kv_head_of``), caches [n_pages, page_size, H_kv, d], block_table
    [B, max_pages], context_lens [B].  A token that sees no key (its position
    below 0) gets O = 0 and LSE = -inf.  Returns (O [B, H, n_q, d], LSE
    [B, H, n_q]) in fp64.

    papermap "FlashAttention-2" explainer, Chapter 03 ("The Downstream
    Story") names paged-KV decoding among the kernels built on
    FlashAttention-2; the page-table indirection (logical key -> physical
    page and slot) is the plain reading of a paged cache, and the result is
    the exact causal attention of the new tokens over the sequence's keys.
    """
    q = _f64(q)
    B, H, n_q, _ = q.shape
    Hkv = np.asarray(k_cache).shape[2]
    o = np.zeros(q.shape[:-1] + (np.asarray(v_cache).shape[3],), dtype=np.float64)
    lse = np.full(q.shape[:-1], -np.inf)
    for b in range(B):
        L = int(context_lens[b])
        mask = visible_decode(n_q, L)
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            kb = gather_pages(k_cache, block_table[b], L, g)
            vb = gather_pages(v_cache, block_table[b], L, g)
            m, l, num = softmax_stats(scores(q[b, h], kb, scale), mask, vb)
            seen = l > 0
            if seen.any():
                o[b, h][seen], lse[b, h][seen] = finalize(m[seen], l[seen], num[seen])
    return o, lse
