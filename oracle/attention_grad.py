"""Plain, slow fp64 CPU oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests and the benchmark's CPU-baseline leg use
it.  It shares no code, tables or helpers with the HIP kernels.

What it computes.  The forward pass is the definition in
``exact_attention``: O = P V with P = softmax(scale * Q K^T) over the visible
keys of each row.  Given the gradient dO of a scalar loss with respect to O,
the chain rule gives, for one head:

    dV  = P^T dO                                   (O is linear in V)
    dP  = dO V^T                                   (O is linear in P)
    dS_i = (diag(P_i) - P_i P_i^T) dP_i            (Jacobian of one softmax row)
         = P_i * (dP_i - sum_j P_ij dP_ij)
    dQ  = scale * dS K                             (S = scale * Q K^T)
    dK  = scale * dS^T Q

Masked entries have P = 0, so they receive no gradient.

Sources.  The pages define only the forward pass; the backward pass appears
as the part of a training step that the headline training numbers include
(Saraf, "FlashAttention 2: Three Places the Chip Was Still Waiting",
section 2.5) and as something a benchmark must say whether it times (Mishra,
"FlashAttention-2 and -3: From Algebra to GPU Scheduling", the benchmarking
checklist).  The reading taken here: the backward pass is the exact gradient
of the forward definition, recomputing P from Q, K and the saved row
statistics rather than storing it (Mishra, the note that a fast kernel may
redo some arithmetic to avoid moving data).  These functions are that
gradient written out with dense fp64 matrices; nothing is tiled.

The identity used by tiled backward passes, sum_j P_ij dP_ij = dO_i . O_i,
is NOT used here: ``grad_scores`` takes the row sum of P * dP directly, and a
pin checks the identity separately.
"""

from __future__ import annotations

import numpy as np

from . import exact_attention as fwd

__all__ = [
    "grad_v",
    "grad_p",
    "grad_scores",
    "grad_q",
    "grad_k",
    "attention_grad_head",
    "attention_grad_ref",
    "attention_grad_ref_gqa",
    "attention_grad_head_window",
    "attention_grad_ref_window",
    "grad_magnitudes_head_window",
    "grad_magnitudes_head",
    "delta_rows",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --- one step of the chain rule per function --------------------------------

def grad_v(p: np.ndarray, dout: np.ndarray) -> np.ndarray:
    """dV = P^T dO: each value row collects the output gradients weighted by
    how much every query attended to it."""
    return p.T @ dout


def grad_p(dout: np.ndarray, v: np.ndarray) -> np.ndarray:
    """dP = dO V^T: gradient with respect to the normalised probabilities."""
    return dout @ v.T


def grad_scores(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS_i = (diag(P_i) - P_i P_i^T) dP_i for every row i (softmax Jacobian).

    Written as P * (dP - rowsum(P * dP)); rows whose keys are all masked have
    P = 0 and get dS = 0.
    """
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def grad_q(ds: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """dQ = scale * dS K."""
    return float(scale) * (ds @ k)


def grad_k(ds: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    """dK = scale * dS^T Q."""
    return float(scale) * (ds.T @ q)


# --- drivers ------------------------------------------------------------------

def attention_grad_head(q, k, v, dout, scale: float, causal: bool):
    """(dQ, dK, dV) of one head, fp64, for q, k, v, dout [N, d].

    P is the normalised probability matrix of the forward definition
    (``exact_attention.probabilities``).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    return _grads_from_p(fwd.probabilities(q, k, scale, causal), q, k, v, dout, scale)


def _grads_from_p(p, q, k, v, dout, scale):
    """The chain rule from the normalised probabilities P of one head."""
    dv = grad_v(p, dout)
    dp = grad_p(dout, v)
    ds = grad_scores(p, dp)
    return grad_q(ds, k, scale), grad_k(ds, q, scale), dv


def attention_grad_head_window(q, k, v, dout, scale: float, window_left: int, window_right: int):
    """(dQ, dK, dV) of one head under a sliding-window mask
    (``exact_attention.visible_window``): the same chain rule, with P from
    ``exact_attention.probabilities_window``."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    return _grads_from_p(fwd.probabilities_window(q, k, scale, window_left, window_right), q, k, v, dout, scale)


def attention_grad_ref_window(q, k, v, dout, scale: float, window_left: int, window_right: int):
    """(dQ, dK, dV) over [B, H, N, d] under a sliding window; k and v may have
    fewer heads (grouped heads: a shared head's gradient is the group sum)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = fwd.kv_head_of(h, H, Hkv)
            gq, gk, gv = attention_grad_head_window(q[b, h], k[b, g], v[b, g], dout[b, h], scale,
                                                    window_left, window_right)
            dq[b, h] = gq
            dk[b, g] += gk
            dv[b, g] += gv
    return dq, dk, dv


def attention_grad_ref(q, k, v, dout, scale: float, causal: bool):
    """(dQ, dK, dV) over [..., N, d] tensors (e.g. [B, H, N, d]), fp64."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for idx in np.ndindex(*q.shape[:-2]):
        dq[idx], dk[idx], dv[idx] = attention_grad_head(q[idx], k[idx], v[idx], dout[idx], scale, causal)
    return dq, dk, dv


def delta_rows(o, dout) -> np.ndarray:
    """D_i = dO_i . O_i over [..., N, d] (the per-row term a tiled backward
    pass precomputes; equal to rowsum(P * dP) by the definition of O)."""
    return (_f64(o) * _f64(dout)).sum(axis=-1)


def grad_magnitudes_head(q, k, v, dout, scale: float, causal: bool):
    """Per-element magnitudes (mQ, mK, mV) of one head for error bounds.

    Each gradient element is a sum of products; its magnitude is the sum of
    the absolute values of those products, with |dS| replaced by a bound that
    also covers the per-row term computed from the forward output:

        |dS|_ij <= P_ij (|dP_ij| + sum_d |dO_id| (P |V|)_id)
        mV = P^T |dO|,   mQ = scale |dS| |K|,   mK = scale |dS|^T |Q|

    A kernel whose only inexact steps are roundings of one factor of each
    product (relative error u) and fp32 accumulation lands within a small
    multiple of u times these magnitudes.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    return _magnitudes_from_p(fwd.probabilities(q, k, scale, causal), q, k, v, dout, scale)


def grad_magnitudes_head_window(q, k, v, dout, scale: float, window_left: int, window_right: int):
    """``grad_magnitudes_head`` under a sliding-window mask."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    return _magnitudes_from_p(fwd.probabilities_window(q, k, scale, window_left, window_right),
                              q, k, v, dout, scale)


def _magnitudes_from_p(p, q, k, v, dout, scale):
    adp = np.abs(grad_p(dout, v))
    row = (np.abs(dout) * (p @ np.abs(v))).sum(axis=1, keepdims=True)
    ads = p * (adp + row)
    return (abs(float(scale)) * (ads @ np.abs(k)), abs(float(scale)) * (ads.T @ np.abs(q)),
            p.T @ np.abs(dout))


def attention_grad_ref_gqa(q, k, v, dout, scale: float, causal: bool):
    """(dQ, dK, dV) with grouped key/value heads: q and dout [B, H, N, d], k
    and v [B, H_kv, N, d].  A key/value head feeds every query head of its
    group, so its gradient is the sum of the per-query-head gradients
    (the adjoint of using one tensor several times)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError(f"{H} query heads cannot share {Hkv} key/value heads evenly")
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = fwd.kv_head_of(h, H, Hkv)
            gq, gk, gv = attention_grad_head(q[b, h], k[b, g], v[b, g], dout[b, h], scale, causal)
            dq[b, h] = gq
            dk[b, g] += gk
            dv[b, g] += gv
    return dq, dk, dv
