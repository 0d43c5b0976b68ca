"""GPU parity of the split forward schedule (fa2_split_plan + fa2_fwd_split).

A query tile's key range cut into chunks, each chunk's partial result
merged by the log-sum weights, must still give the exact attention of the
fp64 oracle within the forward bars (bf16 inputs: |O| <= 1e-2, |LSE| <=
1e-3 with fp32 O; a bf16 O may add half an ulp of the reference).  Every
element is compared on small shapes with chunks of 1, 2, 3 and 5 key tiles
(so rows that see no key of a chunk occur), under causal, full, sliding
windows and grouped heads; the long few-head workload [1, 2, 32768, 128]
causal is checked on sampled rows with the schedule the planner picks.  A
schedule that splits nothing must match the oracle and give what
fa2_fwd_window gives to rounding (fa2_fwd_window runs another kernel, which
rounds exponent arguments and sums in another order).
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


def _check(o, lse, eo, el, what, o_bf16=False):
    o, lse = _np64(o), _np64(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    err_o = np.abs(o - eo)
    err_l = float(np.max(np.abs(lse - el)))
    print(f"[split] {what}: max|dO|={float(np.max(err_o)):.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert np.all(err_o <= 1e-2 + (_bf16_half_ulp(eo) if o_bf16 else 0.0)), what
    assert err_l <= 1e-3, what


CASES = [
    # B, H, H_kv, N, d, window_left, window_right, chunk, outliers, o_bf16
    (1, 2, 2, 700, 128, -1, 0, 1, True, False),
    (1, 2, 2, 700, 128, -1, 0, 3, False, True),
    (1, 1, 1, 1000, 128, -1, -1, 2, False, False),
    (1, 1, 1, 1000, 128, -1, -1, 5, True, True),
    (1, 2, 2, 777, 128, 255, 0, 1, True, False),
    (1, 1, 1, 1000, 128, 128, 128, 2, False, False),
    (1, 1, 1, 600, 128, 300, -1, 3, False, False),
    (1, 2, 1, 513, 64, -1, 0, 1, False, False),
    (1, 2, 1, 513, 64, 77, 20, 2, True, True),
    (2, 4, 2, 300, 128, -1, 0, 1, False, False),
    (1, 1, 1, 2049, 64, -1, 0, 5, False, False),
]


@pytest.mark.parametrize("B,H,H_kv,N,d,wl,wr,chunk,outliers,o_bf16", CASES,
                         ids=[f"{b}x{h}/{hk}x{n}x{d}-w({l},{r})-c{c}{'-bf16o' if ob else ''}"
                              for b, h, hk, n, d, l, r, c, _, ob in CASES])
def test_split_every_element(B, H, H_kv, N, d, wl, wr, chunk, outliers, o_bf16):
    q, k, v = _inputs(B, H, H_kv, N, d, seed=1100 + N + chunk, outliers=outliers)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] split {B}x{H}/{H_kv}x{N}x{d} window=({wl},{wr}) chunk={chunk}", flush=True)
    plan = fa2.split_plan((B, H, N, d), window=(wl, wr), max_chunk_tiles=chunk)
    assert plan.splits
    o_dtype = torch.bfloat16 if o_bf16 else torch.float32
    o, lse = fa2.forward_split(q.to(DEV), k.to(DEV), v.to(DEV), plan, scale=scale, window=(wl, wr),
                               o_dtype=o_dtype)
    torch.cuda.synchronize()
    eo, el = ref.attention_ref_window(_np64(q), _np64(k), _np64(v), scale, wl, wr)
    _check(o, lse, eo, el, f"{B}x{H}/{H_kv}x{N}x{d} w({wl},{wr}) chunk {chunk}", o_bf16)


def test_unsplit_schedule_matches_fa2_fwd_window():
    q, k, v = (t.to(DEV) for t in _inputs(1, 3, 3, 900, 128, seed=21, outliers=True))
    print("[case] unsplit schedule vs fa2_fwd_window", flush=True)
    for window in ((-1, 0), (-1, -1), (100, 30)):
        plan = fa2.split_plan(q.shape, window=window, max_chunk_tiles=10 ** 6)
        assert not plan.splits and plan.workspace_bytes == 0
        o1, l1 = fa2.forward(q, k, v, scale=0.09, window=window)
        o2, l2 = fa2.forward_split(q, k, v, plan, scale=0.09, window=window)
        torch.cuda.synchronize()
        eo, el = ref.attention_ref_window(_np64(q), _np64(k), _np64(v), 0.09, *window)
        _check(o2, l2, eo, el, f"unsplit schedule window={window}")
        d_o = float((o1 - o2).abs().max())
        d_l = float((l1 - l2).abs().max())
        print(f"[split] unsplit vs fa2_fwd_window {window}: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
        assert d_o <= 4e-3 and d_l <= 1e-4, window


def test_split_close_to_unsplit_and_deterministic():
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 2, 1500, 128, seed=22))
    print("[case] split vs unsplit 1x2x1500 causal, chunk 2", flush=True)
    plan = fa2.split_plan(q.shape, causal=True, max_chunk_tiles=2)
    o1, l1 = fa2.forward(q, k, v, causal=True)
    o2, l2 = fa2.forward_split(q, k, v, plan, causal=True)
    o3, l3 = fa2.forward_split(q, k, v, plan, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    d_o = float((o1 - o2).abs().max())
    d_l = float((l1 - l2).abs().max())
    print(f"[split] vs unsplit: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
    assert d_o <= 4e-3 and d_l <= 1e-4


def test_workspace_reuse_across_plans():
    """One workspace serves two schedules in a row (the second smaller):
    nothing of the first call leaks into the second."""
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 2, 1200, 128, seed=23))
    big = fa2.split_plan(q.shape, causal=True, max_chunk_tiles=1)
    ws = torch.full((big.workspace_bytes,), 0x7F, dtype=torch.uint8, device=DEV)
    print("[case] workspace reuse 1x2x1200 causal, chunks 1 then 4", flush=True)
    fa2.forward_split(q, k, v, big, causal=True, workspace=ws)
    q2, k2, v2 = (t.to(DEV) for t in _inputs(1, 2, 2, 700, 128, seed=24))
    small = fa2.split_plan(q2.shape, causal=True, max_chunk_tiles=4)
    assert small.workspace_bytes <= big.workspace_bytes
    o, lse = fa2.forward_split(q2, k2, v2, small, causal=True, workspace=ws)
    torch.cuda.synchronize()
    eo, el = ref.attention_ref(_np64(q2), _np64(k2), _np64(v2), 1.0 / math.sqrt(128), True)
    _check(o, lse, eo, el, "second call on a reused workspace")


def test_long_few_head_planner_schedule_sampled_rows():
    w = workloads.get("long_few_head")
    print(f"[case] split {w.name} {w.shape} causal={w.causal}, planner schedule", flush=True)
    q, k, v = workloads.make_inputs(w, 3, device=DEV)
    plan = fa2.split_plan(q.shape, causal=w.causal)
    print(f"[split] items={plan.n_items} slots={plan.n_slots} workspace={plan.workspace_bytes} B", flush=True)
    assert plan.splits
    o, lse = fa2.forward_split(q, k, v, plan, causal=w.causal, scale=w.scale)
    o1, l1 = fa2.forward(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    d_o = float((o - o1).abs().max())
    d_l = float((lse - l1).abs().max())
    print(f"[split] vs unsplit, all rows: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
    assert d_o <= 4e-3 and d_l <= 1e-4
    rng = np.random.default_rng(31)
    # rows on chunk and tile edges of the split tiles, plus random rows
    rows = {0, 255, 256, w.N - 1, w.N - 256, w.N - 257, w.N // 2, w.N // 2 - 1}
    rows.update(int(r) for r in rng.integers(w.N // 2, w.N, size=24))
    rows = np.array(sorted(rows))
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        eo, el = ref.attention_rows(_np64(q[b, h]), _np64(k[b, h]), _np64(v[b, h]), w.scale, w.causal, rows)
        _check(o[b, h][rows], lse[b, h][rows], eo, el, f"{w.name} head ({b},{h}) {len(rows)} rows")


def test_split_rejections_on_gpu():
    q, k, v = (t.to(DEV) for t in _inputs(1, 1, 1, 600, 128, seed=25))
    plan = fa2.split_plan(q.shape, causal=True, max_chunk_tiles=1)
    small = torch.empty(plan.workspace_bytes - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        fa2.forward_split(q, k, v, plan, causal=True, workspace=small)
    with pytest.raises(ValueError):
        fa2.forward_split(q, k, v, plan, causal=False)  # built for another mask
    with pytest.raises(fa2.Fa2Error):
        fa2.forward_split(q.float(), k.float(), v.float(), plan, causal=True)
