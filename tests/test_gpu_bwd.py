"""GPU parity of the backward pass (d = 128 and d = 64): the HIP path
(through the C ABI) against the fp64 gradient oracle.

Bar (derived in the design notes from the arithmetic): bf16 inputs, P and dS
rounded to bf16 (unit roundoff 2^-9 relative) before the products that use
them, fp32 everywhere else, D computed from the forward's fp32 O (itself
within 2^-9 of the exact O relative to sum_j P_ij |v_j|).  Each gradient
element is a sum of products whose absolute values sum to the oracle's
magnitude m (``grad_magnitudes_head``); the kernel's error is at most about
3 * 2^-9 * m.  The tests require

    |g - g_ref| <= 2^-6 * m + 1e-6 * max(m)

element by element (2^-6 leaves a factor 2.7 over that estimate), plus
bf16 output rounding (half an ulp of the value) when grad_dtype is bf16.

* small shapes spanning several tiles, ragged tails, causal and not: every
  element of dQ, dK, dV;
* the long_causal workload at full size (inputs from the same seeded
  generator the benchmark uses): two whole heads against the oracle, and on
  every head the invariants sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i;
* degenerate cases: N = 1, scale = 0;
* bitwise run-to-run determinism.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_33_amd as fa2
import oracle.attention_grad as gref
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL = 2.0 ** -6


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _fwd_bwd(q, k, v, g, causal, scale, grad_dtype=torch.float32):
    o, lse = fa2.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa2.backward(q, k, v, o, lse, g, causal=causal, scale=scale, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return dq, dk, dv


def _bf16_half_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def _check_head(got, q, k, v, g, scale, causal, what, grad_bf16=False):
    """got: (dq, dk, dv) fp64 [N, d] of one head; q, k, v, g fp64 [N, d]."""
    refs = gref.attention_grad_head(q, k, v, g, scale, causal)
    mags = gref.grad_magnitudes_head(q, k, v, g, scale, causal)
    worst = []
    for name, x, r, m in zip(("dQ", "dK", "dV"), got, refs, mags):
        assert np.all(np.isfinite(x)), f"{what}: non-finite {name}"
        bound = REL * m + 1e-6 * float(np.max(m)) + (_bf16_half_ulp(r) if grad_bf16 else 0.0)
        err = np.abs(x - r)
        ratio = float(np.max(err / np.maximum(m, 1e-30))) if err.size else 0.0
        worst.append(f"{name} max|err|={float(np.max(err)):.3e} max err/m={ratio:.2e}")
        assert np.all(err <= bound), f"{what}: {name} exceeds 2^-6*m ({worst[-1]})"
    print(f"[bwd parity] {what}: " + "; ".join(worst), flush=True)


def _inputs(B, H, N, seed, outliers=False):
    w = workloads.get("long_causal").with_(B=B, H=H, N=N,
                                           outlier_frac=0.001 if outliers else 0.0)
    q, k, v = workloads.make_inputs(w, seed)
    g = workloads.make_grad_output(w, seed + 7919)
    return w, q, k, v, g


SMALL = [
    (1, 2, 127, True, False),
    (1, 2, 127, False, False),
    (2, 1, 256, True, True),
    (1, 3, 300, False, True),
    (1, 1, 200, True, False),
    (1, 1, 33, True, False),
    (1, 2, 520, True, True),
]


@pytest.mark.parametrize("B,H,N,causal,outliers", SMALL,
                         ids=[f"{b}x{h}x{n}-{'causal' if c else 'full'}{'-outl' if o else ''}"
                              for b, h, n, c, o in SMALL])
def test_small_shapes_every_element(B, H, N, causal, outliers):
    w, q, k, v, g = _inputs(B, H, N, seed=1000 + N, outliers=outliers)
    scale = 1.0 / math.sqrt(128)
    print(f"[case] bwd B={B} H={H} N={N} causal={causal} outliers={outliers}", flush=True)
    dq, dk, dv = _fwd_bwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), causal, scale)
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    got = [_np64(t) for t in (dq, dk, dv)]
    for b in range(B):
        for h in range(H):
            _check_head([x[b, h] for x in got], Q[b, h], K[b, h], V[b, h], G[b, h], scale, causal,
                        f"{B}x{H}x{N} causal={causal} head ({b},{h})")


def test_bf16_gradients():
    B, H, N, causal = 1, 2, 300, True
    w, q, k, v, g = _inputs(B, H, N, seed=77, outliers=True)
    scale = 1.0 / math.sqrt(128)
    print("[case] bwd bf16 gradients", flush=True)
    got = _fwd_bwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), causal, scale, grad_dtype=torch.bfloat16)
    assert all(t.dtype == torch.bfloat16 for t in got)
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    got = [_np64(t) for t in got]
    for h in range(H):
        _check_head([x[0, h] for x in got], Q[0, h], K[0, h], V[0, h], G[0, h], scale, causal,
                    f"bf16 grads head {h}", grad_bf16=True)


def test_bf16_forward_output_as_input():
    """o given in bf16 (the forward's o_dtype=bf16): D is computed from it."""
    B, H, N, causal = 1, 2, 256, False
    w, q, k, v, g = _inputs(B, H, N, seed=78)
    scale = 1.0 / math.sqrt(128)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa2.forward(qd, kd, vd, causal=causal, scale=scale, o_dtype=torch.bfloat16)
    dq, dk, dv = fa2.backward(qd, kd, vd, o, lse, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    got = [_np64(t) for t in (dq, dk, dv)]
    # bf16 O adds up to 2^-9 relative to |O| in D; the magnitude's row term
    # (sum_d |dO| P|V|) covers that
    for h in range(H):
        _check_head([x[0, h] for x in got], Q[0, h], K[0, h], V[0, h], G[0, h], scale, causal,
                    f"bf16 O head {h}")


def test_degenerate_single_row_and_zero_scale():
    print("[case] bwd N=1 and scale=0", flush=True)
    # N = 1: P = 1, so dV = dO exactly (P rounds to 1.0 in bf16); dQ and dK
    # are exactly 0 only in exact arithmetic (dP and D are fp32 sums taken in
    # different orders), so they are held to the error bound around 0
    w, q, k, v, g = _inputs(1, 2, 1, seed=3)
    got = _fwd_bwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), True, 0.1)
    dq, dk, dv = (_np64(t) for t in got)
    assert np.array_equal(dv, _np64(g)), "N=1: dV != dO"
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    for h in range(2):
        _check_head([dq[0, h], dk[0, h], dv[0, h]], Q[0, h], K[0, h], V[0, h], G[0, h], 0.1, True,
                    f"N=1 head {h}")
    # scale = 0: uniform attention; the kernels multiply by the scale last,
    # so dQ = dK = 0 exactly
    w, q, k, v, g = _inputs(1, 1, 150, seed=4)
    got = _fwd_bwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), True, 0.0)
    dq, dk, dv = (_np64(t) for t in got)
    assert not np.any(dq) and not np.any(dk), "scale 0: dQ, dK not zero"
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    _check_head([dq[0, 0], dk[0, 0], dv[0, 0]], Q[0, 0], K[0, 0], V[0, 0], G[0, 0], 0.0, True, "scale 0")


def test_deterministic():
    w, q, k, v, g = _inputs(1, 2, 700, seed=5, outliers=True)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    print("[case] bwd determinism", flush=True)
    a = _fwd_bwd(qd, kd, vd, gd, True, 0.088)
    b = _fwd_bwd(qd, kd, vd, gd, True, 0.088)
    for x, y in zip(a, b):
        assert torch.equal(x, y), "backward is not bitwise reproducible"


def test_long_causal_workload():
    """The long_causal workload at full size: two whole heads against the
    oracle, invariants on every head."""
    w = workloads.get("long_causal")
    print("[case] bwd long_causal full size", flush=True)
    q, k, v = workloads.make_inputs(w, 0)
    g = workloads.make_grad_output(w, 7919)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    dq, dk, dv = _fwd_bwd(qd, kd, vd, gd, w.causal, w.scale)
    # invariants on every head, computed on the device in fp64
    sdk = dk.double().sum(dim=2)                      # [B, H, d]
    adk = dk.double().abs().sum(dim=2)
    sdv = dv.double().sum(dim=2)
    sg = gd.double().sum(dim=2)
    adv = dv.double().abs().sum(dim=2)
    assert torch.all(sdk.abs() <= REL * adk + 1e-3), "sum_j dK_j != 0 on some head"
    assert torch.all((sdv - sg).abs() <= REL * adv + 1e-3), "sum_j dV_j != sum_i dO_i on some head"
    Q, K, V, G = (t.double().numpy() for t in (q, k, v, g))
    got = [_np64(t) for t in (dq, dk, dv)]
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        _check_head([x[b, h] for x in got], Q[b, h], K[b, h], V[b, h], G[b, h], w.scale, w.causal,
                    f"long_causal head ({b},{h})")


def test_buffer_rejections_on_gpu():
    """Caller-supplied delta, dq, dk, dv that are host tensors, wrongly sized
    or wrongly typed raise ValueError before any launch."""
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device=DEV)
    o, lse = fa2.forward(q, q, q)
    g = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device=DEV)
    print("[case] bwd buffer rejections", flush=True)
    bad = [
        dict(delta=torch.empty(1, 2, 64)),                                    # host
        dict(delta=torch.empty(1, 2, 63, device=DEV)),                        # short
        dict(delta=torch.empty(1, 2, 64, dtype=torch.bfloat16, device=DEV)),  # dtype
        dict(delta=torch.empty(1, 2, 128, device=DEV)[:, :, ::2]),            # strided
        dict(dq=torch.empty(1, 2, 64, 128)),                                  # host
        dict(dk=torch.empty(1, 2, 64, 64, device=DEV)),                       # shape
        dict(dv=torch.empty(1, 2, 64, 128, dtype=torch.bfloat16, device=DEV)),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            fa2.backward(q, q, q, o, lse, g, **kw)
    torch.cuda.synchronize()


# --- head dimension 64 ------------------------------------------------------
# The same bar; d = 64 has its own LDS layout (rows of 128 bytes, two per
# bank line, with their own chunk permutation) and copy geometry.

SMALL64 = [
    (1, 2, 127, True, False),
    (2, 1, 300, False, True),
    (1, 3, 520, True, True),
    (1, 1, 33, True, False),
    (1, 2, 1000, False, False),
]


def _inputs64(B, H, N, seed, outliers=False):
    w = workloads.get("long_causal").with_(B=B, H=H, N=N, d=64, outlier_frac=0.001 if outliers else 0.0)
    q, k, v = workloads.make_inputs(w, seed)
    g = workloads.make_grad_output(w, seed + 7919)
    return w, q, k, v, g


@pytest.mark.parametrize("B,H,N,causal,outliers", SMALL64,
                         ids=[f"d64-{b}x{h}x{n}-{'causal' if c else 'full'}{'-outl' if o else ''}"
                              for b, h, n, c, o in SMALL64])
def test_d64_every_element(B, H, N, causal, outliers):
    w, q, k, v, g = _inputs64(B, H, N, seed=2000 + N, outliers=outliers)
    scale = 0.125
    print(f"[case] bwd d=64 B={B} H={H} N={N} causal={causal} outliers={outliers}", flush=True)
    dq, dk, dv = _fwd_bwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), causal, scale)
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    got = [_np64(t) for t in (dq, dk, dv)]
    for b in range(B):
        for h in range(H):
            _check_head([x[b, h] for x in got], Q[b, h], K[b, h], V[b, h], G[b, h], scale, causal,
                        f"d64 {B}x{H}x{N} causal={causal} head ({b},{h})")


def test_d64_bf16_gradients_grouped_heads_and_window():
    """d = 64 with bf16 gradients, 4 query heads on 2 key/value heads and a
    window open on both sides, against the window oracle's group sums."""
    B, H, Hkv, N, win = 1, 4, 2, 400, (70, 9)
    w, q, k, v, g = _inputs64(B, H, N, seed=2101, outliers=True)
    k, v = k[:, :Hkv].contiguous(), v[:, :Hkv].contiguous()
    scale = 0.125
    print(f"[case] bwd d=64 bf16 grads, {H}/{Hkv} heads, window {win}", flush=True)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa2.forward(qd, kd, vd, scale=scale, window=win)
    got = fa2.backward(qd, kd, vd, o, lse, gd, scale=scale, window=win, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Q, K, V, G = (_np64(t) for t in (q, k, v, g))
    refs = gref.attention_grad_ref_window(Q, K, V, G, scale, *win)
    mq, mk, mv = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for h in range(H):
        gk = h // (H // Hkv)
        a, bb, c = gref.grad_magnitudes_head_window(Q[0, h], K[0, gk], V[0, gk], G[0, h], scale, *win)
        mq[0, h] = a
        mk[0, gk] += bb
        mv[0, gk] += c
    for name, x, r, m in zip(("dQ", "dK", "dV"), got, refs, (mq, mk, mv)):
        x = _np64(x)
        bound = REL * m + 1e-6 * float(np.max(m)) + _bf16_half_ulp(r)
        err = np.abs(x - r)
        print(f"[bwd parity] d64 window {name}: max|err|={float(np.max(err)):.3e}", flush=True)
        assert np.all(np.isfinite(x)) and np.all(err <= bound), name


def test_d64_deterministic():
    w, q, k, v, g = _inputs64(1, 2, 700, seed=2202, outliers=True)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    print("[case] bwd d=64 determinism", flush=True)
    a = _fwd_bwd(qd, kd, vd, gd, True, 0.125)
    b = _fwd_bwd(qd, kd, vd, gd, True, 0.125)
    for x, y in zip(a, b):
        assert torch.equal(x, y), "backward is not bitwise reproducible"
