"""GPU parity of block-sparse attention (fa2_sparse_plan + fa2_fwd_sparse)
against the fp64 oracle, every element, at the forward bars (bf16 inputs:
|O| <= 1e-2, |LSE| <= 1e-3 with fp32 O; a bf16 O may add half an ulp of
the reference).  Rows that see no key must give exactly O = 0 and
LSE = -inf, as the oracle does.

Masks are seeded random block patterns with blocks of 32 to 512 rows and
64 to 256 keys (so some wavefronts of a tile see a listed key tile and
others do not), causal or not, one mask for all heads, one per head or one
per (sequence, head), with ragged lengths, d = 64 and 128, grouped
key/value heads and bf16 O.  An all-ones mask must give what fa2_fwd gives
to rounding (fa2_fwd runs another kernel, whose exponent arguments and sums
round in another order) and match the oracle, bitwise run to run.  Lists
longer than the kernel's 128-entry register window, sequences up to its
limit of 262,144 keys and one key past it (sampled rows), and LDS-poison
runs (bitwise equal to the ordinary ones) cover the entry window.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_33_amd as fa2
import oracle.exact_attention as ref
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _bf16_half_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def _inputs(B, H, H_kv, N, d, seed, outliers=False):
    w = workloads.get("long_causal").with_(B=B, H=H, N=N, d=d, outlier_frac=0.001 if outliers else 0.0)
    q, k, v = workloads.make_inputs(w, seed)
    return q, k[:, :H_kv].contiguous(), v[:, :H_kv].contiguous()


CASES = [
    # B, H, H_kv, N, d, block_q, block_k, layouts ("one", "head", "all"), density, causal, keep_diag, o_bf16
    (1, 2, 2, 700, 128, 128, 128, "one", 0.4, False, True, False),
    (1, 2, 2, 700, 128, 128, 128, "head", 0.4, True, True, False),
    (2, 2, 1, 1000, 128, 64, 192, "all", 0.3, True, False, False),
    (1, 3, 3, 513, 128, 32, 64, "head", 0.5, False, False, True),
    (1, 2, 2, 777, 64, 256, 128, "one", 0.5, True, True, False),
    (1, 1, 1, 2049, 128, 512, 256, "one", 0.3, True, False, False),
    (2, 4, 2, 300, 64, 96, 64, "all", 0.6, False, False, True),
    (1, 2, 2, 1024, 128, 128, 64, "head", 0.15, False, False, False),
    # past 8192 keys: lists longer than the 128-entry register window, which
    # moves on by 64 entries (once, twice), and key tiles past 255
    (1, 1, 1, 8300, 64, 128, 128, "one", 0.3, True, True, False),
    (1, 1, 1, 9000, 64, 256, 64, "one", 1.0, False, False, False),
    (1, 1, 1, 10000, 128, 256, 128, "one", 1.0, True, False, True),
    (1, 1, 1, 17000, 64, 128, 64, "one", 0.9, True, True, False),
    # long lists with grouped key/value heads, one mask per head or per (b, h)
    (1, 4, 2, 9000, 128, 128, 64, "head", 0.95, True, True, True),
    (2, 2, 1, 8500, 64, 64, 128, "all", 0.8, False, False, False),
]


@pytest.mark.parametrize("B,H,H_kv,N,d,bq,bk,lay,dens,causal,diag,o_bf16", CASES,
                         ids=[f"{b}x{h}/{hk}x{n}x{d}-b{bq}x{bk}-{lay}-p{p}{'-causal' if c else ''}{'-bf16o' if ob else ''}"
                              for b, h, hk, n, d, bq, bk, lay, p, c, _, ob in CASES])
def test_sparse_every_element(B, H, H_kv, N, d, bq, bk, lay, dens, causal, diag, o_bf16):
    q, k, v = _inputs(B, H, H_kv, N, d, seed=1300 + N + bq, outliers=(N % 2 == 1))
    L = {"one": 1, "head": H, "all": B * H}[lay]
    bm = workloads.make_block_mask(L, -(-N // bq), -(-N // bk), dens, seed=N + bk, keep_diagonal=diag)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] sparse {B}x{H}/{H_kv}x{N}x{d} blocks {bq}x{bk} layouts={L} density={dens} "
          f"causal={causal}", flush=True)
    plan = fa2.fa2_sparse_plan(N, bq, bk, bm, causal)
    o_dtype = torch.bfloat16 if o_bf16 else torch.float32
    o, lse = fa2.forward_sparse(q.to(DEV), k.to(DEV), v.to(DEV), plan, scale=scale, o_dtype=o_dtype)
    torch.cuda.synchronize()
    eo, el = ref.attention_ref_block_sparse(_np64(q), _np64(k), _np64(v), scale, bm, bq, bk, causal)
    o, lse = _np64(o), _np64(lse)
    empty = np.isneginf(el)
    print(f"[sparse] empty rows: {int(empty.sum())} of {empty.size}", flush=True)
    assert np.array_equal(np.isneginf(lse), empty), "-inf LSE rows differ from the oracle's empty rows"
    assert np.all(o[empty] == 0.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[~empty]))
    err_o = np.abs(o - eo)
    err_l = float(np.max(np.abs(lse[~empty] - el[~empty]))) if (~empty).any() else 0.0
    print(f"[sparse] max|dO|={float(np.max(err_o)):.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert np.all(err_o <= 1e-2 + (_bf16_half_ulp(eo) if o_bf16 else 0.0))
    assert err_l <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_matches_dense(causal):
    q, k, v = (t.to(DEV) for t in _inputs(1, 3, 3, 900, 128, seed=31, outliers=True))
    print(f"[case] all-ones block mask vs dense, causal={causal}", flush=True)
    bm = np.ones((1, -(-900 // 128), -(-900 // 128)), dtype=bool)
    plan = fa2.fa2_sparse_plan(900, 128, 128, bm, causal)
    o1, l1 = fa2.forward(q, k, v, causal=causal, scale=0.09)
    o2, l2 = fa2.forward_sparse(q, k, v, plan, scale=0.09)
    o3, l3 = fa2.forward_sparse(q, k, v, plan, scale=0.09)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    eo, el = ref.attention_ref(_np64(q), _np64(k), _np64(v), 0.09, causal)
    for o, lse, what in ((o1, l1, "dense"), (o2, l2, "sparse")):
        err_o = float(np.max(np.abs(_np64(o) - eo)))
        err_l = float(np.max(np.abs(_np64(lse) - el)))
        print(f"[sparse] all-ones {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
        assert err_o <= 1e-2 and err_l <= 1e-3, what
    d_o = float((o1 - o2).abs().max())
    d_l = float((l1 - l2).abs().max())
    print(f"[sparse] all-ones vs dense: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
    assert d_o <= 4e-3 and d_l <= 1e-4


def test_empty_mask_gives_zero_and_minus_inf():
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 2, 600, 128, seed=32))
    print("[case] all-zero block mask", flush=True)
    plan = fa2.fa2_sparse_plan(600, 128, 128, np.zeros((1, 5, 5), dtype=bool), True)
    assert plan.n_entries == 0
    o = torch.full(q.shape, 7.0, dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:3], 7.0, dtype=torch.float32, device=DEV)
    fa2.forward_sparse(q, k, v, plan, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0).item() and torch.all(torch.isneginf(lse)).item()


def test_sparse_rejections_on_gpu():
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 2, 600, 128, seed=33))
    plan = fa2.fa2_sparse_plan(600, 128, 128, np.ones((3, 5, 5), dtype=bool), False)  # 3 layouts, 2 heads
    with pytest.raises(fa2.Fa2Error):
        fa2.forward_sparse(q, k, v, plan)
    good = fa2.fa2_sparse_plan(600, 128, 128, np.ones((1, 5, 5), dtype=bool), False)
    with pytest.raises(fa2.Fa2Error):
        fa2.forward_sparse(q.float(), k.float(), v.float(), good)
    with pytest.raises(ValueError):
        fa2.forward_sparse(q[:, :, :500].contiguous(), k[:, :, :500].contiguous(), v[:, :, :500].contiguous(), good)


def test_sparse_headline_size_sampled_rows():
    """long_causal at full size with the masks the benchmark times (one
    seeded mask of 128x128 blocks per head, density 0.3, causal): sampled
    rows of three heads against the oracle's definition."""
    w = workloads.get("long_causal")
    print(f"[case] sparse {w.name} {w.shape} 128x128 blocks p=0.3, sampled rows", flush=True)
    q, k, v = workloads.make_inputs(w, 0, device=DEV)
    nb = -(-w.N // 128)
    bm = workloads.make_block_mask(w.H, nb, nb, 0.3, seed=0)
    plan = fa2.fa2_sparse_plan(w.N, 128, 128, bm, w.causal)
    o, lse = fa2.forward_sparse(q, k, v, plan, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    rows = np.array(sorted({0, 127, 128, 255, 256, w.N - 1, *rng.integers(0, w.N, size=30).tolist()}))
    for b, h in ((0, 0), (1, 15), (1, 4)):
        Q, K, V = _np64(q[b, h]), _np64(k[b, h]), _np64(v[b, h])
        s = ref.scores(Q[rows], K, w.scale)
        vis = ref.visible_block_sparse(rows, np.arange(w.N), bm[h], 128, 128, w.causal)
        m, l, num = ref.softmax_stats(s, vis, V)
        eo, el = ref.finalize(m, l, num)
        err_o = float(np.max(np.abs(_np64(o[b, h][rows]) - eo)))
        err_l = float(np.max(np.abs(_np64(lse[b, h][rows]) - el)))
        print(f"[sparse] head ({b},{h}): max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
        assert err_o <= 1e-2 and err_l <= 1e-3


def test_sparse_long_lists_sampled_rows():
    """40,000 keys at d = 128 (625 key tiles; lists of up to ~470 entries, so
    the register window moves on several times within an item), two heads
    with their own masks of 128x128 blocks at density 0.75, causal: sampled
    rows, among them the first and last of 128-row halves deep in the
    sequence, against the oracle's definition."""
    N, H, bq, bk, dens = 40000, 2, 128, 128, 0.75
    q, k, v = (t.to(DEV) for t in _inputs(1, H, H, N, 128, seed=41, outliers=True))
    print(f"[case] sparse 1x{H}x{N}x128 blocks {bq}x{bk} p={dens} causal, sampled rows", flush=True)
    nb = -(-N // bq)
    bm = workloads.make_block_mask(H, nb, -(-N // bk), dens, seed=42)
    plan = fa2.fa2_sparse_plan(N, bq, bk, bm, True)
    scale = 1.0 / math.sqrt(128)
    o, lse = fa2.forward_sparse(q, k, v, plan, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    rows = np.array(sorted({0, 31, 32, 127, 128, 20000 - 1, 20000, 32767, 32768, N - 129, N - 128, N - 1,
                            *rng.integers(0, N, size=24).tolist()}))
    for h in range(H):
        Q, K, V = _np64(q[0, h]), _np64(k[0, h]), _np64(v[0, h])
        s = ref.scores(Q[rows], K, scale)
        vis = ref.visible_block_sparse(rows, np.arange(N), bm[h], bq, bk, True)
        m, l, num = ref.softmax_stats(s, vis, V)
        eo, el = ref.finalize(m, l, num)
        ob, lb = _np64(o[0, h][rows]), _np64(lse[0, h][rows])
        empty = np.isneginf(el)
        assert np.array_equal(np.isneginf(lb), empty) and np.all(ob[empty] == 0.0)
        err_o = float(np.max(np.abs(ob - eo)))
        err_l = float(np.max(np.abs(lb[~empty] - el[~empty]))) if (~empty).any() else 0.0
        print(f"[sparse] head {h}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
        assert err_o <= 1e-2 and err_l <= 1e-3


@pytest.mark.parametrize("N", [262144, 262145])
def test_sparse_length_limit_sampled_rows(N):
    """At the 128-row kernel's limit of 4,096 key tiles (262,144 keys: key
    tile 4,095 is the largest its 12-bit entries hold) and one key past it
    (the 256-row kernel): one head, d = 64, a mask of 256x64 blocks at
    density 0.1, not causal (lists of ~410 entries), sampled rows against
    the oracle's definition."""
    bq, bk, dens = 256, 64, 0.1
    q, k, v = (t.to(DEV) for t in _inputs(1, 1, 1, N, 64, seed=43))
    print(f"[case] sparse 1x1x{N}x64 blocks {bq}x{bk} p={dens}, sampled rows", flush=True)
    bm = workloads.make_block_mask(1, -(-N // bq), -(-N // bk), dens, seed=44, keep_diagonal=False)
    plan = fa2.fa2_sparse_plan(N, bq, bk, bm, False)
    o, lse = fa2.forward_sparse(q, k, v, plan, scale=0.125)
    torch.cuda.synchronize()
    rng = np.random.default_rng(19)
    rows = np.array(sorted({0, 127, 128, 255, 256, N - 257, N - 129, N - 128, N - 1,
                            *rng.integers(0, N, size=20).tolist()}))
    Q, K, V = _np64(q[0, 0]), _np64(k[0, 0]), _np64(v[0, 0])
    s = ref.scores(Q[rows], K, 0.125)
    vis = ref.visible_block_sparse(rows, np.arange(N), bm[0], bq, bk, False)
    assert vis[:, -64:].any(), "no sampled row sees the last key tile"
    m, l, num = ref.softmax_stats(s, vis, V)
    eo, el = ref.finalize(m, l, num)
    ob, lb = _np64(o[0, 0][rows]), _np64(lse[0, 0][rows])
    err_o = float(np.max(np.abs(ob - eo)))
    err_l = float(np.max(np.abs(lb - el)))
    print(f"[sparse] N={N}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= 1e-2 and err_l <= 1e-3


SPARSE_POISON = [(1000, 128, 128, 64, 0.5, True), (9000, 64, 256, 64, 1.0, False), (10000, 128, 256, 128, 1.0, True)]


@pytest.mark.parametrize("N,d,bq,bk,dens,causal", SPARSE_POISON,
                         ids=[f"{n}x{d}-b{bq}x{bk}-p{p}{'-causal' if c else ''}" for n, d, bq, bk, p, c in SPARSE_POISON])
def test_sparse_lds_poison(monkeypatch, N, d, bq, bk, dens, causal):
    """With FA2_DEBUG_POISON the kernel fills each K/V ring slot with NaN
    before a tile is copied into it: a read ahead of a copy, a copy over a
    slot still being read, or a list entry kept where the ring lives would
    change O.  The result must be bitwise that of the ordinary run (lists
    of up to 157 entries, so the window moves on)."""
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 2, N, d, seed=45, outliers=True))
    print(f"[case] sparse poisoned LDS 1x2x{N}x{d} blocks {bq}x{bk} p={dens} causal={causal}", flush=True)
    bm = workloads.make_block_mask(2, -(-N // bq), -(-N // bk), dens, seed=46, keep_diagonal=False)
    plan = fa2.fa2_sparse_plan(N, bq, bk, bm, causal)
    o0, l0 = fa2.forward_sparse(q, k, v, plan, scale=0.1)
    monkeypatch.setenv("FA2_DEBUG_POISON", "1")
    o1, l1 = fa2.forward_sparse(q, k, v, plan, scale=0.1)
    monkeypatch.delenv("FA2_DEBUG_POISON")
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    if N <= 1000:
        eo, el = ref.attention_ref_block_sparse(_np64(q), _np64(k), _np64(v), 0.1, bm, bq, bk, causal)
        empty = np.isneginf(el)
        assert np.array_equal(np.isneginf(_np64(l1)), empty)
        assert float(np.max(np.abs(_np64(o1) - eo))) <= 1e-2
        assert float(np.max(np.abs(_np64(l1)[~empty] - el[~empty]))) <= 1e-3
