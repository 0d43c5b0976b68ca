"""The FP8 oracle against its pins, and planted mistakes it must catch."""

import math

import numpy as np
import pytest

import oracle.fp8_attention as f8
from oracle_fp8_pins import FP8_PINS

_orig_rotate = f8.rotate_fp32
_orig_encode = f8.e4m3_encode
_orig_values = f8.e4m3_values
_orig_quant = f8.quantize_block


@pytest.mark.parametrize("pin", FP8_PINS, ids=[p.__name__ for p in FP8_PINS])
def test_fp8_pin(pin):
    pin()


def _encode_round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    grid = _orig_values()[:127]
    ax = np.abs(x).reshape(-1)
    idx = np.clip(np.searchsorted(grid, ax), 1, 126)
    lo, hi = grid[idx - 1], grid[idx]
    code = np.where(ax - lo >= hi - ax, idx, idx - 1)
    code = np.where(ax == 0, 0, code).reshape(x.shape) | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def _encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    grid = _orig_values()[:127]
    ax = np.abs(x).reshape(-1)
    code = np.clip(np.searchsorted(grid, ax, side="right") - 1, 0, 126)
    return (code.reshape(x.shape) | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _values_bias8():
    v = _orig_values()
    return v / 2.0


def _values_subnormal_wrong():
    v = _orig_values().copy()
    for c in range(1, 8):
        v[c] = c * 2.0 ** -10
        v[0x80 | c] = -c * 2.0 ** -10
    return v


def _rotate_no_scale(x, s):
    return _orig_rotate(x, s) * np.float32(math.sqrt(np.asarray(x).shape[-1]))


def _rotate_no_signs(x, s):
    return _orig_rotate(x, np.ones_like(np.asarray(s)))


def _rotate_sign_only(x, s):
    return (np.asarray(x, dtype=np.float32) * np.asarray(s, dtype=np.float32))


def _quant_scale_inverted(x32):
    codes, sc = _orig_quant(x32)
    return codes, np.float32(1.0 / sc) if sc != 0 else sc


def _quant_amax_of_signed(x32):
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(x32)) if x32.size else np.float32(0)
    if amax <= 0:
        return np.zeros(x32.shape, dtype=np.uint8), np.float32(1.0)
    y = np.clip(x32 * (np.float32(448) / amax), -448, 448)
    return _orig_encode(y), np.float32(amax / np.float32(448))


MUTANTS = {
    "encode_round_half_up": ("e4m3_encode", _encode_round_half_up),
    "encode_truncate": ("e4m3_encode", _encode_truncate),
    "values_exponent_bias_8": ("e4m3_values", _values_bias8),
    "values_subnormal_spacing": ("e4m3_values", _values_subnormal_wrong),
    "rotate_without_1_over_sqrt_d": ("rotate_fp32", _rotate_no_scale),
    "rotate_without_signs": ("rotate_fp32", _rotate_no_signs),
    "rotate_sign_flip_only": ("rotate_fp32", _rotate_sign_only),
    "quantize_scale_inverted": ("quantize_block", _quant_scale_inverted),
    "quantize_amax_signed": ("quantize_block", _quant_amax_of_signed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(f8, attr, fn)
    caught = []
    for pin in FP8_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every FP8 pin"
