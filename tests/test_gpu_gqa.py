"""GPU parity of grouped key/value heads (GQA, and MQA with one key/value
head): fa2_fwd_gqa and fa2_bwd_gqa against the fp64 oracles.

Bars: the forward ones (bf16 inputs: |O| <= 1e-2, |LSE| <= 1e-3 with fp32
O; fp32 inputs: both <= 1e-5) and the backward one (|g - g_ref| <= 2^-6 m +
1e-6 max(m), m the per-element magnitude; for a shared key/value head, dK
and dV are sums over the group and so are their magnitudes).  Every element
is compared.  With H_kv = H the grouped entry points must give bitwise the
results of fa2_fwd / fa2_bwd.
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


def _inputs(B, H, H_kv, N, d, dtype, seed, outliers=False):
    w = workloads.get("long_causal").with_(B=B, H=H, N=N, d=d, dtype=dtype,
                                           outlier_frac=0.001 if outliers else 0.0)
    q, k, v = workloads.make_inputs(w, seed)
    g = workloads.make_grad_output(w, seed + 7919)
    return q, k[:, :H_kv].contiguous(), v[:, :H_kv].contiguous(), g


FWD = [
    (1, 8, 2, 300, 128, "bf16", True, True),
    (2, 4, 1, 257, 128, "bf16", False, False),
    (1, 6, 3, 520, 64, "bf16", True, False),
    (1, 4, 2, 100, 64, "fp32", True, False),
    (1, 4, 4, 130, 128, "bf16", True, False),
    # unmasked, B*H a multiple of 8 (XCD-major tile order with grouped heads)
    (2, 8, 2, 600, 128, "bf16", False, True),
    (1, 16, 4, 300, 64, "bf16", False, False),
]


@pytest.mark.parametrize("B,H,H_kv,N,d,dtype,causal,outliers", FWD,
                         ids=[f"{b}x{h}/{hk}x{n}x{d}-{t}-{'causal' if c else 'full'}" for b, h, hk, n, d, t, c, _ in FWD])
def test_gqa_forward_every_element(B, H, H_kv, N, d, dtype, causal, outliers):
    q, k, v, _ = _inputs(B, H, H_kv, N, d, dtype, seed=400 + N, outliers=outliers)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] gqa fwd {B}x{H}/{H_kv}x{N}x{d} {dtype} causal={causal}", flush=True)
    o, lse = fa2.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    eo, el = ref.attention_ref_gqa(_np64(q), _np64(k), _np64(v), scale, causal)
    to, tl = (1e-2, 1e-3) if dtype == "bf16" else (1e-5, 1e-5)
    err_o = float(np.max(np.abs(_np64(o) - eo)))
    err_l = float(np.max(np.abs(_np64(lse) - el)))
    print(f"[gqa fwd] max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= to and err_l <= tl


def test_gqa_with_all_heads_equals_multi_head_bitwise():
    q, k, v, g = _inputs(1, 4, 4, 333, 128, "bf16", seed=9, outliers=True)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    B, H, N, d = q.shape
    o1 = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    l1 = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    h = torch.cuda.current_stream().cuda_stream
    assert fa2.fa2_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(), l1.data_ptr(),
                       B, H, N, d, 1, 0.09, h, fa2.BF16, fa2.F32) == fa2.FA2_OK
    assert fa2.fa2_fwd_gqa(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                           B, H, H, N, d, 1, 0.09, h, fa2.BF16, fa2.F32) == fa2.FA2_OK
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    a = fa2.backward(qd, kd, vd, o1, l1, gd, causal=True, scale=0.09)
    outs = [torch.empty(q.shape, dtype=torch.float32, device=DEV) for _ in range(3)]
    delta = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    assert fa2.fa2_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(), gd.data_ptr(),
                       l1.data_ptr(), delta.data_ptr(), *(t.data_ptr() for t in outs), B, H, N, d, 1,
                       0.09, h, fa2.BF16, fa2.F32, fa2.F32) == fa2.FA2_OK
    torch.cuda.synchronize()
    for x, y in zip(a, outs):
        assert torch.equal(x, y)


BWD = [
    (1, 4, 2, 300, True, True),
    (1, 4, 1, 200, False, False),
    (2, 6, 3, 130, True, False),
]


@pytest.mark.parametrize("B,H,H_kv,N,causal,outliers", BWD,
                         ids=[f"{b}x{h}/{hk}x{n}-{'causal' if c else 'full'}" for b, h, hk, n, c, _ in BWD])
def test_gqa_backward_every_element(B, H, H_kv, N, causal, outliers):
    q, k, v, g = _inputs(B, H, H_kv, N, 128, "bf16", seed=600 + N, outliers=outliers)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] gqa bwd {B}x{H}/{H_kv}x{N} causal={causal}", flush=True)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa2.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa2.backward(qd, kd, vd, o, lse, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    rq, rk, rv = gref.attention_grad_ref_gqa(Q, K, V, G, scale, causal)
    mq = np.zeros_like(Q)
    mk = np.zeros_like(K)
    mv = np.zeros_like(V)
    group = H // H_kv
    for b in range(B):
        for h in range(H):
            gk = h // group
            a, bb, c = gref.grad_magnitudes_head(Q[b, h], K[b, gk], V[b, gk], G[b, h], scale, causal)
            mq[b, h] = a
            mk[b, gk] += bb
            mv[b, gk] += c
    for name, x, r, m in (("dQ", dq, rq, mq), ("dK", dk, rk, mk), ("dV", dv, rv, mv)):
        x = _np64(x)
        err = np.abs(x - r)
        ratio = float(np.max(err / np.maximum(m, 1e-30)))
        print(f"[gqa bwd] {name}: max|err|={float(np.max(err)):.3e} max err/m={ratio:.2e}", flush=True)
        assert np.all(err <= 2.0 ** -6 * m + 1e-6 * float(np.max(m))), f"{name} exceeds the bound"


def test_gqa_headline_size_sampled_rows():
    """long_causal at full size with 4 key/value heads (the configuration
    `bench.py --kv-heads 4` times): sampled rows of three query heads,
    each against its group's key/value head."""
    w = workloads.get("long_causal")
    print(f"[case] gqa fwd {w.name} {w.shape} with 4 key/value heads, sampled rows", flush=True)
    q, k, v = workloads.make_inputs(w, 0, device=DEV)
    k, v = k[:, :4].contiguous(), v[:, :4].contiguous()
    o, lse = fa2.forward(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(14)
    rows = np.array(sorted({0, 255, 256, w.N - 1, *rng.integers(0, w.N, size=30).tolist()}))
    for b, h in ((0, 0), (1, 15), (0, 6)):
        g = ref.kv_head_of(h, w.H, 4)
        eo, el = ref.attention_rows(_np64(q[b, h]), _np64(k[b, g]), _np64(v[b, g]), w.scale, True, rows)
        err_o = float(np.max(np.abs(_np64(o[b, h][rows]) - eo)))
        err_l = float(np.max(np.abs(_np64(lse[b, h][rows]) - el)))
        print(f"[gqa fwd] head ({b},{h}) -> kv {g}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
        assert err_o <= 1e-2 and err_l <= 1e-3
