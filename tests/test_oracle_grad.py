"""The fp64 gradient oracle against its pins, an independent autograd
rendering, and planted mistakes (CPU only)."""

import numpy as np
import pytest
import torch

import oracle.attention_grad as gref
from oracle_grad_pins import GRAD_PINS


@pytest.mark.parametrize("pin", GRAD_PINS, ids=[p.__name__ for p in GRAD_PINS])
def test_grad_pin(pin):
    pin()


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_float64_autograd(causal):
    """torch autograd through masked_fill + softmax in float64 (a separate
    implementation of the forward definition) gives the same gradients."""
    rng = np.random.default_rng(31)
    b, h, n, d = 2, 3, 45, 16
    arrs = [rng.normal(size=(b, h, n, d)) for _ in range(4)]
    scale = 0.27
    q, k, v = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in arrs[:3])
    g = torch.tensor(arrs[3], dtype=torch.float64)
    s = scale * (q @ k.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ v
    o.backward(g)
    dq, dk, dv = gref.attention_grad_ref(*arrs, scale, causal)
    np.testing.assert_allclose(dq, q.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, k.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, v.grad.numpy(), atol=1e-12, rtol=0)


_orig = {name: getattr(gref, name) for name in ("grad_v", "grad_p", "grad_scores", "grad_q", "grad_k")}


def _gqa_last_head_wins(q, k, v, dout, scale, causal):
    """Planted mistake: a shared key/value head keeps only its last query
    head's gradient instead of the sum."""
    import oracle.exact_attention as fwd

    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    dq, dk, dv = np.empty_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = fwd.kv_head_of(h, H, Hkv)
            dq[b, h], dk[b, g], dv[b, g] = gref.attention_grad_head(q[b, h], k[b, g], v[b, g], dout[b, h], scale, causal)
    return dq, dk, dv


_orig_grad_window = gref.attention_grad_ref_window
_orig_mag_window = gref.grad_magnitudes_head_window


def _window_grad_driver(head_of, accumulate=True):
    """A copy of the [B, H] window gradient driver: query head h reads
    key/value head head_of(h, H, H_kv); accumulate=False stores a shared
    head's gradient instead of adding it (the last query head wins)."""
    def driver(q, k, v, dout, scale, wl, wr):
        q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        B, H = q.shape[:2]
        Hkv = k.shape[1]
        dq, dk, dv = np.empty_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                g = head_of(h, H, Hkv)
                gq, gk, gv = gref.attention_grad_head_window(q[b, h], k[b, g], v[b, g], dout[b, h], scale, wl, wr)
                dq[b, h] = gq
                if accumulate:
                    dk[b, g] += gk
                    dv[b, g] += gv
                else:
                    dk[b, g] = gk
                    dv[b, g] = gv
        return dq, dk, dv
    return driver


MUTANTS = {
    "grad_v_untransposed_p": ("grad_v", lambda p, dout: p @ dout if p.shape[0] == dout.shape[0] else p.T @ dout + 1),
    "grad_v_sign": ("grad_v", lambda p, dout: -(p.T @ dout)),
    "grad_p_transposed": ("grad_p", lambda dout, v: (dout @ v.T).T if dout.shape[0] == v.shape[0] else dout @ v.T + 1),
    "grad_p_sign": ("grad_p", lambda dout, v: -(dout @ v.T)),
    "grad_scores_no_rowsum": ("grad_scores", lambda p, dp: p * dp),
    "grad_scores_colsum": ("grad_scores", lambda p, dp: p * (dp - (p * dp).sum(axis=0, keepdims=True))),
    "grad_scores_rowsum_of_dp": ("grad_scores", lambda p, dp: p * (dp - dp.sum(axis=1, keepdims=True))),
    "grad_scores_not_times_p": ("grad_scores", lambda p, dp: dp - (p * dp).sum(axis=1, keepdims=True)),
    "grad_q_no_scale": ("grad_q", lambda ds, k, scale: ds @ k),
    "grad_q_transposed_ds": ("grad_q", lambda ds, k, scale: float(scale) * (ds.T @ k)),
    "grad_k_untransposed_ds": ("grad_k", lambda ds, q, scale: float(scale) * (ds @ q)),
    "grad_k_sign": ("grad_k", lambda ds, q, scale: -float(scale) * (ds.T @ q)),
    "gqa_last_head_wins": ("attention_grad_ref_gqa", _gqa_last_head_wins),
    "window_grad_driver_sides_swapped": ("attention_grad_ref_window", lambda q, k, v, g, s, wl, wr: _orig_grad_window(
        q, k, v, g, s, wr, wl)),
    "window_grad_driver_assigns": ("attention_grad_ref_window", _window_grad_driver(
        lambda h, n_h, n_kv: h // (n_h // n_kv), accumulate=False)),
    "window_grad_driver_heads_interleaved": ("attention_grad_ref_window", _window_grad_driver(
        lambda h, n_h, n_kv: h % n_kv)),
    "window_grad_driver_heads_ungrouped": ("attention_grad_ref_window", _window_grad_driver(lambda h, n_h, n_kv: h)),
    "window_magnitudes_sides_swapped": ("grad_magnitudes_head_window", lambda q, k, v, g, s, wl, wr: _orig_mag_window(
        q, k, v, g, s, wr, wl)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_grad_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(gref, attr, fn)
    caught = []
    for pin in GRAD_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__ + " (error)")
    assert caught, f"mutant {name} passed every gradient pin"
