"""Pins of the fp64 gradient oracle against facts other than the oracle itself.

Each ``pin_*`` function raises AssertionError when ``oracle.attention_grad``
disagrees with what the mathematics fixes:

* central finite differences of the forward definition, evaluated by explicit
  Python loops with ``math.fsum`` (no code shared with the gradient oracle);
* closed forms (one key; zero scale; two keys and one query);
* invariants that hold for any input (sum over keys of dK is zero, sum over
  keys of dV equals the sum over queries of dO, sum Q*dQ equals sum K*dK);
* the row identity rowsum(P * dP) = dO . O that tiled backward passes use.

``test_oracle_grad.py`` runs them and shows that planted mistakes in every
step of the gradient oracle make at least one fail.  All pins look the oracle
up through the module object at call time, so a monkeypatched step is seen.
"""

from __future__ import annotations

import math

import numpy as np

import oracle.attention_grad as gref
import oracle.exact_attention as ref


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _loss_loops(q, k, v, g, scale, causal):
    """sum_i sum_c g_ic O_ic with O from the definition, by explicit loops."""
    n, d, dv = len(q), len(q[0]), len(v[0])
    total = []
    for i in range(n):
        keys = [j for j in range(len(k)) if (not causal) or j <= i]
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(w.values())
        for c in range(dv):
            total.append(g[i][c] * math.fsum(w[j] * v[j][c] for j in keys) / den)
    return math.fsum(total)


def _finite_difference(q, k, v, g, scale, causal, h=1e-6):
    """Central differences of the loop loss with respect to every input entry."""
    grads = []
    for which in range(3):
        base = [q, k, v][which]
        out = np.zeros_like(base)
        for idx in np.ndindex(*base.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            up = _loss_loops(*(a.tolist() for a in args), g.tolist(), scale, causal)
            args[which][idx] -= 2 * h
            dn = _loss_loops(*(a.tolist() for a in args), g.tolist(), scale, causal)
            out[idx] = (up - dn) / (2 * h)
        grads.append(out)
    return grads


def pin_grad_finite_differences():
    """Random tiny heads: oracle gradients == central finite differences."""
    rng = _rng(2024)
    for trial in range(12):
        n = int(rng.integers(1, 6))
        d = int(rng.integers(1, 4))
        dv = int(rng.integers(1, 4))
        q, k = rng.normal(size=(n, d)), rng.normal(size=(n, d))
        v, g = rng.normal(size=(n, dv)), rng.normal(size=(n, dv))
        scale = float(rng.choice([0.3, 1.0, 1.7]))
        for causal in (False, True):
            fq, fk, fv = _finite_difference(q, k, v, g, scale, causal)
            dq, dk, dvv = gref.attention_grad_head(q, k, v, g, scale, causal)
            tag = f"trial {trial} n={n} d={d} causal={causal}"
            _close(dq, fq, 2e-8, "FD dQ " + tag)
            _close(dk, fk, 2e-8, "FD dK " + tag)
            _close(dvv, fv, 2e-8, "FD dV " + tag)


def pin_grad_single_key():
    """N = 1: P = 1, so dV = dO and the scores get no gradient."""
    rng = _rng(5)
    for causal in (False, True):
        q, k, v, g = (rng.normal(size=(1, 6)) for _ in range(4))
        dq, dk, dv = gref.attention_grad_head(q, k, v, g, 0.8, causal)
        _close(dv, g, 1e-15, f"N=1 dV causal={causal}")
        _close(dq, np.zeros_like(q), 1e-15, f"N=1 dQ causal={causal}")
        _close(dk, np.zeros_like(k), 1e-15, f"N=1 dK causal={causal}")


def pin_grad_zero_scale():
    """scale = 0: uniform attention over the visible keys, so
    dV_j = sum over the queries that see key j of dO_i / (number of keys i
    sees), and dQ = dK = 0."""
    rng = _rng(6)
    n, d = 7, 3
    q, k, v, g = (rng.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = gref.attention_grad_head(q, k, v, g, 0.0, causal)
        expect = np.zeros((n, d))
        for i in range(n):
            keys = range(i + 1) if causal else range(n)
            for j in keys:
                expect[j] += g[i] / len(keys)
        _close(dv, expect, 1e-14, f"scale 0 dV causal={causal}")
        _close(dq, np.zeros_like(q), 0.0, f"scale 0 dQ causal={causal}")
        _close(dk, np.zeros_like(k), 0.0, f"scale 0 dK causal={causal}")


def pin_grad_two_keys_closed_form():
    """One query, two keys (non-causal): with p1 = 1 / (1 + exp(s2 - s1)),
    dS1 = -dS2 = p1 p2 (dO.v1 - dO.v2), dQ = scale dS1 (k1 - k2),
    dK1 = scale dS1 q, dK2 = -dK1, dV_j = p_j dO."""
    rng = _rng(8)
    for trial in range(5):
        q = rng.normal(size=(1, 4))
        k = rng.normal(size=(2, 4))
        v = rng.normal(size=(2, 3))
        g = rng.normal(size=(1, 3))
        # keys 0 and 1 both visible to the single query only when non-causal
        scale = 0.9
        s1, s2 = scale * float(q[0] @ k[0]), scale * float(q[0] @ k[1])
        p1 = 1.0 / (1.0 + math.exp(s2 - s1))
        p2 = 1.0 - p1
        ds1 = p1 * p2 * (float(g[0] @ v[0]) - float(g[0] @ v[1]))
        qq = np.vstack([q, q])  # two identical queries: each sees both keys
        gg = np.vstack([g, np.zeros_like(g)])
        dq, dk, dv = gref.attention_grad_head(qq, k, v, gg, scale, False)
        _close(dq[0], scale * ds1 * (k[0] - k[1]), 1e-14, f"two keys dQ trial {trial}")
        _close(dq[1], np.zeros(4), 1e-15, f"two keys dQ (zero dO row) trial {trial}")
        _close(dk[0], scale * ds1 * q[0], 1e-14, f"two keys dK1 trial {trial}")
        _close(dk[1], -scale * ds1 * q[0], 1e-14, f"two keys dK2 trial {trial}")
        _close(dv, np.vstack([p1 * g[0], p2 * g[0]]), 1e-14, f"two keys dV trial {trial}")


def pin_grad_invariants():
    """For any input: sum_j dK_j = 0 (each row of dS sums to zero);
    sum_j dV_j = sum_i dO_i (each row of P sums to one);
    sum Q*dQ = sum K*dK (S depends on Q and K only through their product)."""
    rng = _rng(9)
    n, d = 37, 16
    q, k = rng.normal(size=(n, d)) * 1.5, rng.normal(size=(n, d)) * 1.5
    v, g = rng.normal(size=(n, d)), rng.normal(size=(n, d))
    for causal in (False, True):
        dq, dk, dv = gref.attention_grad_head(q, k, v, g, 0.35, causal)
        scale_ref = np.abs(dk).max()
        _close(dk.sum(axis=0), np.zeros(d), 1e-12 * max(1.0, scale_ref) * n, f"sum dK causal={causal}")
        _close(dv.sum(axis=0), g.sum(axis=0), 1e-11, f"sum dV causal={causal}")
        _close(np.sum(q * dq), np.sum(k * dk), 1e-10, f"Q.dQ = K.dK causal={causal}")


def pin_delta_identity():
    """rowsum(P * dP) equals dO_i . O_i with O from the forward oracle."""
    rng = _rng(10)
    n, d = 29, 8
    q, k, v, g = (rng.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        o, _ = ref.attention_head(q, k, v, 0.5, causal)
        p = ref.probabilities(q, k, 0.5, causal)
        dp = gref.grad_p(g, v)
        _close(gref.delta_rows(o, g), (p * dp).sum(axis=1), 1e-12, f"D identity causal={causal}")


def pin_magnitudes_bound_gradients():
    """The error-bound magnitudes dominate the gradients they bound."""
    rng = _rng(12)
    n, d = 21, 8
    q, k, v, g = (rng.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        grads = gref.attention_grad_head(q, k, v, g, 0.6, causal)
        mags = gref.grad_magnitudes_head(q, k, v, g, 0.6, causal)
        for name, gr, mg in zip("QKV", grads, mags):
            assert np.all(np.abs(gr) <= mg * (1 + 1e-12) + 1e-300), f"|d{name}| exceeds its magnitude"


def pin_gqa_grad_finite_differences():
    """Grouped key/value heads (4 query heads on 2, and on 1): gradients with
    respect to the shared K and V equal central finite differences of the
    loss summed over all query heads, each evaluated by explicit loops on
    the key/value head it reads (0, 0, 1, 1 and 0, 0, 0, 0)."""
    rng = _rng(2025)
    n, d = 4, 2
    for hkv, groups in ((2, [0, 0, 1, 1]), (1, [0, 0, 0, 0])):
        q = rng.normal(size=(1, 4, n, d))
        k, v = rng.normal(size=(1, hkv, n, d)), rng.normal(size=(1, hkv, n, d))
        g = rng.normal(size=(1, 4, n, d))
        for causal in (False, True):
            def loss(kk, vv, qq=q):
                return math.fsum(_loss_loops(qq[0, h].tolist(), kk[0, groups[h]].tolist(),
                                             vv[0, groups[h]].tolist(), g[0, h].tolist(), 0.7, causal)
                                 for h in range(4))
            h_ = 1e-6
            fk, fv = np.zeros_like(k), np.zeros_like(v)
            for idx in np.ndindex(*k.shape):
                kp, km = k.copy(), k.copy()
                kp[idx] += h_
                km[idx] -= h_
                fk[idx] = (loss(kp, v) - loss(km, v)) / (2 * h_)
                vp, vm = v.copy(), v.copy()
                vp[idx] += h_
                vm[idx] -= h_
                fv[idx] = (loss(k, vp) - loss(k, vm)) / (2 * h_)
            fq = np.zeros_like(q)
            for idx in np.ndindex(*q.shape):
                qp, qm = q.copy(), q.copy()
                qp[idx] += h_
                qm[idx] -= h_
                fq[idx] = (loss(k, v, qp) - loss(k, v, qm)) / (2 * h_)
            dq, dk, dv = gref.attention_grad_ref_gqa(q, k, v, g, 0.7, causal)
            tag = f"H_kv={hkv} causal={causal}"
            _close(dq, fq, 2e-8, "GQA FD dQ " + tag)
            _close(dk, fk, 2e-8, "GQA FD dK " + tag)
            _close(dv, fv, 2e-8, "GQA FD dV " + tag)


def _loss_loops_window(q, k, v, g, scale, wl, wr):
    """sum_i g_i . O_i under a sliding window, by explicit loops."""
    n, d, dv = len(q), len(q[0]), len(v[0])
    total = []
    for i in range(n):
        keys = [j for j in range(len(k)) if (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)]
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(w.values())
        for c in range(dv):
            total.append(g[i][c] * math.fsum(w[j] * v[j][c] for j in keys) / den)
    return math.fsum(total)


def pin_window_grad_finite_differences():
    """Sliding windows: gradients == central finite differences of the
    loop-evaluated loss."""
    rng = _rng(2026)
    h = 1e-6
    for trial, (wl, wr) in enumerate(((1, 0), (2, 1), (0, 0), (-1, 1), (1, -1))):
        n = 5
        q, k, v, g = (rng.normal(size=(n, 2)) for _ in range(4))
        ref_grads = gref.attention_grad_head_window(q, k, v, g, 0.9, wl, wr)
        for which in range(3):
            base = [q, k, v][which]
            fd = np.zeros_like(base)
            for idx in np.ndindex(*base.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                up = _loss_loops_window(*(a.tolist() for a in args), g.tolist(), 0.9, wl, wr)
                args[which][idx] -= 2 * h
                dn = _loss_loops_window(*(a.tolist() for a in args), g.tolist(), 0.9, wl, wr)
                fd[idx] = (up - dn) / (2 * h)
            _close(ref_grads[which], fd, 2e-8, f"window ({wl},{wr}) FD d{'QKV'[which]}")


def pin_window_grad_driver_grouped_heads():
    """The [B, H] sliding-window gradient driver with 4 query heads on 2
    key/value heads (heads 0, 0, 1, 1) and on 1, windows that differ on the
    two sides: dQ, dK, dV equal central finite differences of the loss summed
    over the query heads, each head evaluated by explicit loops on the
    key/value head it reads -- so a shared head's gradient is the sum over
    its group."""
    rng = _rng(2027)
    n, d, h_ = 4, 2, 1e-6
    for hkv, groups in ((2, [0, 0, 1, 1]), (1, [0, 0, 0, 0])):
        q = rng.normal(size=(1, 4, n, d))
        k, v = rng.normal(size=(1, hkv, n, d)), rng.normal(size=(1, hkv, n, d))
        g = rng.normal(size=(1, 4, n, d))
        for wl, wr in ((2, 0), (0, 1), (-1, 1)):
            def loss(qq, kk, vv):
                return math.fsum(_loss_loops_window(qq[0, h].tolist(), kk[0, groups[h]].tolist(),
                                                    vv[0, groups[h]].tolist(), g[0, h].tolist(), 0.8, wl, wr)
                                 for h in range(4))
            ref_grads = gref.attention_grad_ref_window(q, k, v, g, 0.8, wl, wr)
            for which in range(3):
                base = [q, k, v][which]
                fd = np.zeros_like(base)
                for idx in np.ndindex(*base.shape):
                    args = [q.copy(), k.copy(), v.copy()]
                    args[which][idx] += h_
                    up = loss(*args)
                    args[which][idx] -= 2 * h_
                    fd[idx] = (up - loss(*args)) / (2 * h_)
                _close(ref_grads[which], fd, 2e-8, f"window driver H_kv={hkv} ({wl},{wr}) FD d{'QKV'[which]}")


def pin_window_magnitudes():
    """The window error-bound magnitudes: equal to the causal / unmasked ones
    for the windows (-1, 0) and (-1, -1); closed forms for the window (0, 0)
    (each row sees only its own key, P = I) and for two keys under (1, 0)
    (row 0 sees key 0, row 1 sees keys 0 and 1 with P_10 = 1/(1+e^(S11-S10)));
    and they bound the window gradients."""
    rng = _rng(13)
    n, d = 9, 4
    q, k, v, g = (rng.normal(size=(n, d)) for _ in range(4))
    for (wl, wr), causal in (((-1, 0), True), ((-1, -1), False)):
        for a, b_ in zip(gref.grad_magnitudes_head_window(q, k, v, g, 0.5, wl, wr),
                         gref.grad_magnitudes_head(q, k, v, g, 0.5, causal)):
            _close(a, b_, 1e-13, f"magnitudes ({wl},{wr}) vs causal={causal}")
    mq, mk, mv = gref.grad_magnitudes_head_window(q, k, v, g, 0.5, 0, 0)
    ds = np.abs(np.einsum("id,id->i", g, v)) + np.einsum("id,id->i", np.abs(g), np.abs(v))
    _close(mv, np.abs(g), 1e-14, "(0,0) mV = |dO|")
    _close(mq, 0.5 * ds[:, None] * np.abs(k), 1e-13, "(0,0) mQ")
    _close(mk, 0.5 * ds[:, None] * np.abs(q), 1e-13, "(0,0) mK")
    q2, k2, v2, g2 = q[:2], k[:2], v[:2], g[:2]
    s10, s11 = 0.5 * float(q2[1] @ k2[0]), 0.5 * float(q2[1] @ k2[1])
    p10 = 1.0 / (1.0 + math.exp(s11 - s10))
    _, _, mv2 = gref.grad_magnitudes_head_window(q2, k2, v2, g2, 0.5, 1, 0)
    _close(mv2[0], np.abs(g2[0]) + p10 * np.abs(g2[1]), 1e-14, "(1,0) two keys: mV_0")
    _close(mv2[1], (1.0 - p10) * np.abs(g2[1]), 1e-14, "(1,0) two keys: mV_1")
    for wl, wr in ((2, 0), (1, 3), (-1, 1)):
        grads = gref.attention_grad_head_window(q, k, v, g, 0.5, wl, wr)
        mags = gref.grad_magnitudes_head_window(q, k, v, g, 0.5, wl, wr)
        for name, gr, mg in zip("QKV", grads, mags):
            assert np.all(np.abs(gr) <= mg * (1 + 1e-12) + 1e-300), f"({wl},{wr}) |d{name}| exceeds its magnitude"


GRAD_PINS = [
    pin_window_grad_finite_differences,
    pin_window_grad_driver_grouped_heads,
    pin_window_magnitudes,
    pin_gqa_grad_finite_differences,
    pin_grad_finite_differences,
    pin_grad_single_key,
    pin_grad_zero_scale,
    pin_grad_two_keys_closed_form,
    pin_grad_invariants,
    pin_delta_identity,
    pin_magnitudes_bound_gradients,
]
