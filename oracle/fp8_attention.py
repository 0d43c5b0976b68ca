"""Plain CPU oracle for the FP8 forward pass with incoherent processing.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests and the benchmark's CPU-baseline leg use
it.  It shares no code, tables or helpers with the HIP kernels.

What it computes (Mishra, "FlashAttention-2 and -3: From Algebra to GPU
Scheduling", "Low precision changes numerical error"): quantizing Q and K
to FP8 loses information that fp32 accumulation cannot restore, and how
much depends on block scaling and on outliers; a shared orthogonal mixing
transform R applied to both before quantizing leaves the scores unchanged
in exact arithmetic, (QR)(KR)^T = QK^T, while spreading an outlier over
all coordinates (a sign flip alone would not: it keeps every magnitude).

Readings (the pages fix none of the details):
  * R = diag(signs) H / sqrt(d) with H the d x d Sylvester-Hadamard matrix
    (entries +-1, H H^T = d I) and `signs` a +-1 vector: a mixing transform
    (every output coordinate depends on every input coordinate), orthogonal.
  * The product x R is computed in fp32 exactly as written here: signs
    applied (exact), then the butterfly stages h = 1, 2, 4, ..., d/2, each
    replacing (a, b) at positions (i, i + h) of every block of 2h by
    (a + b, a - b) in fp32, then one fp32 multiply by the fp32 constant
    1/sqrt(d).  The quantized codes depend on these fp32 values, so the
    order is part of the definition.
  * FP8 is OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    largest finite 448, subnormals down to 2^-9, no infinities).  Encoding
    rounds to the nearest representable value, ties to the even code.
  * One scale per (sequence, head) block of rotated Q (and of rotated K):
    amax = max |x R| over the block, inv = 448 / amax in fp32, codes =
    E4M3(clamp(x R * inv, -448, 448)) with the product in fp32; the value of
    a code is decode(code) * amax / 448 (amax = 0: all codes 0, scale 1).
  * V stays bf16; attention is then computed exactly (fp64) on the
    dequantized rotated Q and K.
"""

from __future__ import annotations

import math

import numpy as np

from . import exact_attention as ex

__all__ = [
    "hadamard_matrix",
    "rotate_fp32",
    "e4m3_values",
    "e4m3_encode",
    "e4m3_decode",
    "quantize_block",
    "pack_fp8",
    "attention_ref_fp8",
    "score_error_bound",
]

E4M3_MAX = 448.0


def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester-Hadamard matrix of order d (a power of two), fp64:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError(f"d = {d} is not a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_fp32(x, signs) -> np.ndarray:
    """x R in fp32 by the butterfly order stated in the module docstring;
    x [..., d] (any float dtype, converted to fp32 exactly for bf16 inputs),
    signs [d] of +-1."""
    y = (np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)).copy()
    d = y.shape[-1]
    h = 1
    while h < d:
        shape = y.shape[:-1] + (d // (2 * h), 2, h)
        z = y.reshape(shape)
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b  # fp32 + fp32 -> fp32
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y * np.float32(1.0 / math.sqrt(d))


def e4m3_values() -> np.ndarray:
    """Value of every code 0..255 (fp64; NaN for the two NaN codes), from
    the format's definition."""
    out = np.empty(256)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = s * m * 2.0 ** -9
        else:
            out[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_decode(codes) -> np.ndarray:
    return e4m3_values()[np.asarray(codes, dtype=np.int64)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (|x| <= 448), ties to the even code,
    the sign bit set for negative inputs (a negative value that rounds to
    zero gives -0, code 0x80); by search over the 127 non-negative finite
    codes."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("E4M3 encoding takes finite values of magnitude <= 448")
    grid = e4m3_values()[:127]            # codes 0..126: 0, subnormals, normals up to 448
    ax = np.abs(x).reshape(-1)
    idx = np.searchsorted(grid, ax)       # grid[idx-1] < ax <= grid[idx]
    idx = np.clip(idx, 1, 126)
    lo, hi = grid[idx - 1], grid[idx]
    pick_hi = (ax - lo > hi - ax) | ((ax - lo == hi - ax) & (idx % 2 == 0))
    code = np.where(pick_hi, idx, idx - 1)
    code = np.where(ax == 0.0, 0, code).reshape(x.shape)
    # the sign bit follows the input's sign, also for values that round to 0
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def quantize_block(x32) -> tuple[np.ndarray, np.float32]:
    """Codes and scale (amax / 448, fp32) of one block of fp32 values."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    if amax == 0.0:
        return np.zeros(x32.shape, dtype=np.uint8), np.float32(1.0)
    inv = np.float32(E4M3_MAX) / amax                       # fp32 division
    y = np.clip(x32 * inv, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(y), np.float32(amax / np.float32(E4M3_MAX))


def pack_fp8(x, signs, rotate: bool = True):
    """Codes [B, H, N, d] (uint8) and scales [B, H] (fp32) of x [B, H, N, d]
    after the rotation (or, rotate=False, of x itself in fp32)."""
    x = np.asarray(x)
    y = rotate_fp32(x, signs) if rotate else np.asarray(x, dtype=np.float32)
    codes = np.empty(y.shape, dtype=np.uint8)
    scales = np.empty(y.shape[:2], dtype=np.float32)
    for b in range(y.shape[0]):
        for h in range(y.shape[1]):
            codes[b, h], scales[b, h] = quantize_block(y[b, h])
    return codes, scales


def attention_ref_fp8(q, k, v, scale: float, causal: bool, signs, rotate: bool = True):
    """The FP8 forward pass: Q and K packed as above (k, v may have fewer
    heads: grouped heads), then exact fp64 attention of the dequantized
    codes with V.  Returns (O, LSE) in fp64."""
    qc, qs = pack_fp8(q, signs, rotate)
    kc, ks = pack_fp8(k, signs, rotate)
    qd = e4m3_decode(qc) * qs.astype(np.float64)[:, :, None, None]
    kd = e4m3_decode(kc) * ks.astype(np.float64)[:, :, None, None]
    return ex.attention_ref_gqa(qd, kd, np.asarray(v, dtype=np.float64), scale, causal)


def score_error_bound(q, k, scale: float, causal: bool, signs, rotate: bool = True) -> np.ndarray:
    """Per-row bound [B, H, N] on |S_fp8 - S_exact| over visible keys, from
    the quantization alone: every code's value is within max(2^-4 |x|,
    2^-10 s) of the fp32 value it encodes (3 mantissa bits, RNE; subnormal
    spacing 2^-9 s), plus an allowance of 2^-20 |x| for the fp32 rotation's
    own rounding (orders of magnitude below the quantization term), so
        |dS_ij| <= scale * sum_d (|q_d| e(k_d) + e(q_d) |k_d| + e(q_d) e(k_d))
    with e(x) the per-value error bound and q, k the rotated fp32 values."""
    q32 = rotate_fp32(q, signs) if rotate else np.asarray(q, dtype=np.float32)
    k32 = rotate_fp32(k, signs) if rotate else np.asarray(k, dtype=np.float32)
    _, qs = pack_fp8(q, signs, rotate)
    _, ks = pack_fp8(k, signs, rotate)
    B, H, N, _ = q32.shape
    Hkv = k32.shape[1]
    out = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            g = ex.kv_head_of(h, H, Hkv)
            aq = np.abs(q32[b, h]).astype(np.float64)
            ak = np.abs(k32[b, g]).astype(np.float64)
            eq = np.maximum(2.0 ** -4 * aq, 2.0 ** -10 * float(qs[b, h])) + 2.0 ** -20 * aq
            ek = np.maximum(2.0 ** -4 * ak, 2.0 ** -10 * float(ks[b, g])) + 2.0 ** -20 * ak
            bound = abs(scale) * (aq @ ek.T + eq @ ak.T + eq @ ek.T)
            vis = ex.visible(np.arange(N), np.arange(N), causal)
            out[b, h] = np.where(vis, bound, 0.0).max(axis=1)
    return out
