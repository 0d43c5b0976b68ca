"""GPU parity of sliding-window (local) attention: fa2_fwd_window and
fa2_bwd_window against the fp64 oracles, every element, at the forward bars
(bf16 inputs: |O| <= 1e-2, |LSE| <= 1e-3 with fp32 O) and the backward one
(|g - g_ref| <= 2^-6 m + 1e-6 max(m), m the per-element magnitude).

Windows are chosen to land on and around the 64-key tile and 256-row query
tile edges, one-sided and two-sided, with ragged sequence lengths, d = 64
and d = 128, and grouped key/value heads.  The causal window (-1, 0) and
the unbounded one (-1, -1) must give bitwise what fa2_fwd gives.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_33_amd as fa2
import oracle.attention_grad as gref
import oracle.exact_attention as ref
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _inputs(B, H, H_kv, N, d, seed, outliers=False):
    w = workloads.get("long_causal").with_(B=B, H=H, N=N, d=d, outlier_frac=0.001 if outliers else 0.0)
    q, k, v = workloads.make_inputs(w, seed)
    return q, k[:, :H_kv].contiguous(), v[:, :H_kv].contiguous()


CASES = [
    # B, H, H_kv, N, d, window_left, window_right, outliers
    (1, 2, 2, 700, 128, 0, 0, False),
    (1, 2, 2, 700, 128, 63, 0, False),
    (1, 2, 2, 700, 128, 64, 0, True),
    (1, 2, 2, 700, 128, 100, 0, False),
    (1, 2, 2, 777, 128, 255, 0, True),
    (1, 2, 2, 777, 128, 256, 0, False),
    (1, 1, 1, 1000, 128, 128, 128, False),
    (1, 1, 1, 1000, 128, 50, 200, True),
    (1, 1, 1, 600, 128, -1, 100, False),
    (1, 1, 1, 600, 128, 300, -1, False),
    (1, 2, 1, 513, 64, 77, 0, False),
    (2, 4, 2, 300, 128, 31, 5, True),
    (1, 1, 1, 129, 128, 5000, 0, False),
]


@pytest.mark.parametrize("B,H,H_kv,N,d,wl,wr,outliers", CASES,
                         ids=[f"{b}x{h}/{hk}x{n}x{d}-w({l},{r})" for b, h, hk, n, d, l, r, _ in CASES])
def test_window_every_element(B, H, H_kv, N, d, wl, wr, outliers):
    q, k, v = _inputs(B, H, H_kv, N, d, seed=800 + N + wl, outliers=outliers)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] window fwd {B}x{H}/{H_kv}x{N}x{d} window=({wl},{wr})", flush=True)
    o, lse = fa2.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, window=(wl, wr))
    torch.cuda.synchronize()
    eo, el = ref.attention_ref_window(_np64(q), _np64(k), _np64(v), scale, wl, wr)
    o, lse = _np64(o), _np64(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    err_o = float(np.max(np.abs(o - eo)))
    err_l = float(np.max(np.abs(lse - el)))
    print(f"[window fwd] max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= 1e-2 and err_l <= 1e-3


def test_causal_and_unbounded_windows_are_bitwise_the_plain_masks():
    q, k, v = (t.to(DEV) for t in _inputs(1, 3, 3, 900, 128, seed=12, outliers=True))
    print("[case] window (-1,0) / (-1,-1) vs causal / full", flush=True)
    for causal, window in ((True, (-1, 0)), (False, (-1, -1)), (True, (2000, 0))):
        o1, l1 = fa2.forward(q, k, v, causal=causal, scale=0.09)
        o2, l2 = fa2.forward(q, k, v, scale=0.09, window=window)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), window


def test_window_rejections():
    q, k, v = (t.to(DEV) for t in _inputs(1, 1, 1, 64, 128, seed=13))
    with pytest.raises(fa2.Fa2Error):
        fa2.forward(q, k, v, window=(-2, 0))
    qf, kf, vf = (t.float() for t in (q, k, v))
    with pytest.raises(fa2.Fa2Error):
        fa2.forward(qf, kf, vf, window=(10, 0))   # fp32: no mask or causal only


# --- backward under a sliding window ------------------------------------------

BWD = [
    # B, H, H_kv, N, window_left, window_right, outliers
    (1, 2, 2, 700, 63, 0, True),
    (1, 1, 1, 600, 100, 50, False),
    (1, 2, 1, 513, 77, 0, False),
    (1, 1, 1, 1000, 128, 128, False),
    (1, 1, 1, 600, -1, 100, False),
    (1, 1, 1, 600, 300, -1, True),
    (2, 4, 2, 300, 31, 5, False),
    (1, 1, 1, 200, 0, 0, False),
]


@pytest.mark.parametrize("B,H,H_kv,N,wl,wr,outliers", BWD,
                         ids=[f"{b}x{h}/{hk}x{n}-w({l},{r})" for b, h, hk, n, l, r, _ in BWD])
def test_window_backward_every_element(B, H, H_kv, N, wl, wr, outliers):
    q, k, v = _inputs(B, H, H_kv, N, 128, seed=900 + N + wl, outliers=outliers)
    w = workloads.get("long_causal").with_(B=B, H=H, N=N)
    g = workloads.make_grad_output(w, 901 + N)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] window bwd {B}x{H}/{H_kv}x{N} window=({wl},{wr})", flush=True)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa2.forward(qd, kd, vd, scale=scale, window=(wl, wr))
    dq, dk, dv = fa2.backward(qd, kd, vd, o, lse, gd, scale=scale, window=(wl, wr))
    torch.cuda.synchronize()
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    refs = gref.attention_grad_ref_window(Q, K, V, G, scale, wl, wr)
    mq, mk, mv = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    group = H // H_kv
    for b in range(B):
        for h in range(H):
            gk = h // group
            a, bb, c = gref.grad_magnitudes_head_window(Q[b, h], K[b, gk], V[b, gk], G[b, h], scale, wl, wr)
            mq[b, h] = a
            mk[b, gk] += bb
            mv[b, gk] += c
    for name, x, r, m in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs, (mq, mk, mv)):
        x = _np64(x)
        assert np.all(np.isfinite(x)), name
        err = np.abs(x - r)
        ratio = float(np.max(err / np.maximum(m, 1e-30)))
        print(f"[window bwd] {name}: max|err|={float(np.max(err)):.3e} max err/m={ratio:.2e}", flush=True)
        assert np.all(err <= 2.0 ** -6 * m + 1e-6 * float(np.max(m))), f"{name} exceeds the bound"


def test_causal_window_backward_is_bitwise_the_causal_backward():
    q, k, v = (t.to(DEV) for t in _inputs(1, 2, 2, 640, 128, seed=14, outliers=True))
    g = workloads.make_grad_output(workloads.get("long_causal").with_(B=1, H=2, N=640), 15).to(DEV)
    print("[case] window bwd (-1,0) vs causal", flush=True)
    o, lse = fa2.forward(q, k, v, causal=True, scale=0.09)
    a = fa2.backward(q, k, v, o, lse, g, causal=True, scale=0.09)
    b = fa2.backward(q, k, v, o, lse, g, scale=0.09, window=(-1, 0))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_window_headline_size_sampled_rows():
    """long_causal at full size under the (4095, 0) window the benchmark
    times: sampled rows of three heads against the oracle's definition."""
    w = workloads.get("long_causal")
    wl, wr = 4095, 0
    print(f"[case] window fwd {w.name} {w.shape} window=({wl},{wr}), sampled rows", flush=True)
    q, k, v = workloads.make_inputs(w, 0, device=DEV)
    o, lse = fa2.forward(q, k, v, scale=w.scale, window=(wl, wr))
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.array(sorted({0, 4095, 4096, 4097, w.N - 1, *rng.integers(0, w.N, size=30).tolist()}))
    for b, h in ((0, 0), (1, 15), (0, 9)):
        Q, K, V = _np64(q[b, h]), _np64(k[b, h]), _np64(v[b, h])
        s = ref.scores(Q[rows], K, w.scale)
        m, l, num = ref.softmax_stats(s, ref.visible_window(rows, np.arange(w.N), wl, wr), V)
        eo, el = ref.finalize(m, l, num)
        err_o = float(np.max(np.abs(_np64(o[b, h][rows]) - eo)))
        err_l = float(np.max(np.abs(_np64(lse[b, h][rows]) - el)))
        print(f"[window fwd] head ({b},{h}): max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
        assert err_o <= 1e-2 and err_l <= 1e-3
