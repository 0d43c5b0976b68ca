"""Pins of the FP8 oracle (``oracle.fp8_attention``) against facts other
than the oracle itself: the Hadamard matrix's definition, the E4M3 format's
definition, exactly representable cases and the quantization error bound.
Collected in FP8_PINS; ``test_oracle_fp8.py`` runs them and shows that
planted mistakes fail at least one."""

from __future__ import annotations

import math

import numpy as np

import oracle.exact_attention as ex
import oracle.fp8_attention as f8


def _rng(seed):
    return np.random.default_rng(seed)


def pin_hadamard_orthogonal():
    """H H^T = d I exactly; R = diag(s) H / sqrt(d) is orthogonal, so
    (Q R)(K R)^T = Q K^T (Mishra, "Low precision changes numerical error")."""
    for d in (1, 2, 4, 8, 64, 128):
        h = f8.hadamard_matrix(d)
        assert np.array_equal(h @ h.T, d * np.eye(d)), d
        assert set(np.unique(h)) <= {-1.0, 1.0}
    rng = _rng(61)
    d = 64
    s = rng.choice([-1.0, 1.0], size=d)
    r = np.diag(s) @ f8.hadamard_matrix(d) / math.sqrt(d)
    assert np.max(np.abs(r @ r.T - np.eye(d))) <= 1e-14
    q, k = rng.normal(size=(9, d)), rng.normal(size=(7, d))
    assert np.max(np.abs((q @ r) @ (k @ r).T - q @ k.T)) <= 1e-12


def pin_rotation_matches_matrix():
    """rotate_fp32 is x diag(s) H / sqrt(d): within fp32 rounding for random
    inputs, and exactly (one final rounding) for small integers, whose
    butterfly sums are exact in fp32."""
    rng = _rng(62)
    for d in (64, 128):
        s = rng.choice([-1.0, 1.0], size=d)
        r = np.diag(s) @ f8.hadamard_matrix(d) / math.sqrt(d)
        x = rng.normal(size=(5, d)).astype(np.float32)
        y = f8.rotate_fp32(x, s)
        assert y.dtype == np.float32
        ref = x.astype(np.float64) @ r
        assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(x)) * math.sqrt(d)
        xi = rng.integers(-1000, 1001, size=(5, d)).astype(np.float32)
        exact = (xi.astype(np.float64) * s) @ f8.hadamard_matrix(d)   # integers, exact
        want = exact.astype(np.float32) * np.float32(1.0 / math.sqrt(d))
        assert np.array_equal(f8.rotate_fp32(xi, s), want)


def pin_mixing_spreads_an_outlier():
    """A lone outlier coordinate is spread evenly over all d coordinates by
    R; a sign flip alone keeps its magnitude."""
    d = 128
    s = _rng(63).choice([-1.0, 1.0], size=d)
    x = np.zeros((1, d), dtype=np.float32)
    x[0, 5] = 100.0
    y = f8.rotate_fp32(x, s)
    assert np.allclose(np.abs(y), 100.0 / math.sqrt(d), rtol=1e-6)
    assert np.max(np.abs(x * s)) == 100.0


def pin_e4m3_format():
    """E4M3: largest finite 448, smallest normal 2^-6, smallest subnormal
    2^-9, two NaN codes, values increasing over codes 0..126; every finite
    value encodes to its own code (both signs); midpoints go to the even
    code, points just off them to the nearer value."""
    v = f8.e4m3_values()
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    assert np.all(np.diff(v[:127]) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    codes = np.arange(127)
    assert np.array_equal(f8.e4m3_encode(v[codes]), codes.astype(np.uint8))
    assert np.array_equal(f8.e4m3_encode(-v[1:127]), (np.arange(1, 127) | 0x80).astype(np.uint8))
    for c in range(126):
        mid = (v[c] + v[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert f8.e4m3_encode(np.array([mid]))[0] == even, c
        assert f8.e4m3_encode(np.array([np.nextafter(mid, 0)]))[0] == c
        assert f8.e4m3_encode(np.array([np.nextafter(mid, 1e9)]))[0] == c + 1
    assert f8.e4m3_encode(np.array([-1e-6]))[0] == 0x80


def pin_quantize_bound():
    """Each dequantized value is within max(2^-4 |x|, 2^-10 s) of x (RNE with
    3 mantissa bits; subnormal spacing 2^-9 s); the block's largest
    magnitude maps to +-448."""
    rng = _rng(64)
    for trial in range(5):
        x = (rng.normal(size=(37, 16)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        x[3, 4] *= 50.0
        codes, sc = f8.quantize_block(x)
        deq = f8.e4m3_decode(codes) * float(sc)
        err = np.abs(deq - x)
        assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * float(sc)) * (1 + 1e-6)), trial
        i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert abs(f8.e4m3_decode(codes[i])) == 448.0
    codes, sc = f8.quantize_block(np.zeros((4, 4), dtype=np.float32))
    assert np.all(codes == 0) and sc == 1.0


def pin_fp8_attention_exact_inputs():
    """Unrotated Q and K already on the E4M3 grid with block maximum 448
    quantize exactly, so the FP8 pass equals exact attention."""
    rng = _rng(65)
    grid = f8.e4m3_values()[:127]
    B, H, N, d = 1, 2, 9, 16
    q = rng.choice(grid[40:100], size=(B, H, N, d)) * rng.choice([-1, 1], size=(B, H, N, d))
    k = rng.choice(grid[40:100], size=(B, H, N, d)) * rng.choice([-1, 1], size=(B, H, N, d))
    q[:, :, 0, 0] = 448.0
    k[:, :, 0, 0] = -448.0
    v = rng.normal(size=(B, H, N, d))
    for causal in (False, True):
        o, lse = f8.attention_ref_fp8(q, k, v, 0.001, causal, np.ones(d), rotate=False)
        eo, el = ex.attention_ref_gqa(q, k, v, 0.001, causal)
        assert np.max(np.abs(o - eo)) <= 1e-12 and np.max(np.abs(lse - el)) <= 1e-12


def pin_score_bound_holds():
    """The per-row bound of score_error_bound covers the actual score error
    of the quantized, rotated Q and K, with and without outliers."""
    rng = _rng(66)
    B, H, N, d = 1, 2, 40, 64
    s = rng.choice([-1.0, 1.0], size=d)
    for outliers in (False, True):
        q = rng.normal(size=(B, H, N, d)).astype(np.float32)
        k = rng.normal(size=(B, H, N, d)).astype(np.float32)
        if outliers:
            q[rng.random(q.shape) < 0.01] *= 20
            k[rng.random(k.shape) < 0.01] *= 20
        for rotate in (True, False):
            qc, qs = f8.pack_fp8(q, s, rotate)
            kc, ks = f8.pack_fp8(k, s, rotate)
            qd = f8.e4m3_decode(qc) * float(qs[0, 0])
            bound = f8.score_error_bound(q, k, 0.125, True, s, rotate)
            for h in range(H):
                qd = f8.e4m3_decode(qc[0, h]) * float(qs[0, h])
                kd = f8.e4m3_decode(kc[0, h]) * float(ks[0, h])
                err = np.abs(0.125 * (qd @ kd.T) - 0.125 * (q[0, h].astype(np.float64) @ k[0, h].astype(np.float64).T))
                vis = ex.visible(np.arange(N), np.arange(N), True)
                assert np.all(np.where(vis, err, 0.0).max(axis=1) <= bound[0, h]), (outliers, rotate, h)


def pin_pack_layout():
    """pack_fp8 quantizes each (sequence, head) block on its own."""
    rng = _rng(67)
    x = rng.normal(size=(2, 3, 5, 8)).astype(np.float32)
    x[1, 2] *= 100.0
    s = rng.choice([-1.0, 1.0], size=8)
    codes, scales = f8.pack_fp8(x, s, True)
    y = f8.rotate_fp32(x, s)
    for b in range(2):
        for h in range(3):
            c, sc = f8.quantize_block(y[b, h])
            assert np.array_equal(codes[b, h], c) and scales[b, h] == sc


FP8_PINS = [
    pin_hadamard_orthogonal,
    pin_rotation_matches_matrix,
    pin_mixing_spreads_an_outlier,
    pin_e4m3_format,
    pin_quantize_bound,
    pin_fp8_attention_exact_inputs,
    pin_score_bound_holds,
    pin_pack_layout,
]
