"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant replaces one step function of ``oracle.attention_ref`` (on the
CPU, for the duration of one test) with a plausibly wrong version: a
dropped term, a wrong sign or index, a transposed operand, a wrong mask.
The test passes only if the pin suite catches it -- evidence that the pins
constrain every step of the oracle, not just that the oracle agrees with
itself.
"""

import numpy as np
import pytest

import oracle.exact_attention as ref
from oracle_pins import PINS

_orig_scores = ref.scores
_orig_visible = ref.visible
_orig_stats = ref.softmax_stats
_orig_finalize = ref.finalize
_orig_visible_window = ref.visible_window
_orig_visible_bs = ref.visible_block_sparse
_orig_gather = ref.gather_pages
_orig_ref_window = ref.attention_ref_window
_orig_probs_window = ref.probabilities_window


def _probs_window_all_keys(q, k, scale, wl, wr):
    # plausible mistake: the band masks the numerator but the sum runs over all keys
    s = ref.scores(q, k, scale)
    mask = ref.visible_window(np.arange(len(q)), np.arange(len(k)), wl, wr)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return np.where(mask, e, 0.0) / e.sum(axis=1, keepdims=True)


def _probs_window_columns(q, k, scale, wl, wr):
    # plausible mistake: normalised over the query axis
    p = _orig_probs_window(q, k, scale, wl, wr)
    num = p * _orig_probs_window(q, k, scale, wl, wr).sum(axis=1, keepdims=True)
    return num / np.maximum(num.sum(axis=0, keepdims=True), 1e-300)


def _window_driver_heads(head_of):
    """A copy of the [B, H] window driver whose query head h reads the
    key/value head head_of(h, H, H_kv)."""
    def driver(q, k, v, scale, wl, wr):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H = q.shape[:2]
        Hkv = k.shape[1]
        o = np.empty(q.shape[:-1] + (v.shape[-1],))
        lse = np.empty(q.shape[:-1])
        for b in range(B):
            for h in range(H):
                g = head_of(h, H, Hkv)
                o[b, h], lse[b, h] = ref.attention_head_window(q[b, h], k[b, g], v[b, g], scale, wl, wr)
        return o, lse
    return driver


def _stats_no_shift(s, mask, v):
    p = np.where(mask, np.exp(s), 0.0)
    m = np.zeros(s.shape[0])
    return m, p.sum(axis=1), p @ v


def _stats_mask_ignored_in_l(s, mask, v):
    m, _, num = _orig_stats(s, mask, v)
    l = np.exp(s - np.where(np.isfinite(m), m, 0.0)[:, None]).sum(axis=1)
    return m, l, num


def _stats_exp2(s, mask, v):
    s_vis = np.where(mask, s, -np.inf)
    m = s_vis.max(axis=1)
    p = np.where(mask, np.exp2(s - m[:, None]), 0.0)
    return m, p.sum(axis=1), p @ v


def _stats_reversed_v(s, mask, v):
    return _orig_stats(s, mask, v[::-1])


def _stats_m_from_all_keys(s, mask, v):
    m = s.max(axis=1)
    p = np.where(mask, np.exp(s - m[:, None]), 0.0)
    return m, p.sum(axis=1), p @ v


MUTANTS = {
    "scores_transposed": ("scores", lambda q, k, scale: float(scale) * (k @ q.T)
                          if q.shape == k.shape else float(scale) * (q @ k.T) + 1.0),
    "scores_scale_dropped": ("scores", lambda q, k, scale: q @ k.T),
    "scores_scale_squared": ("scores", lambda q, k, scale: float(scale) ** 2 * (q @ k.T)),
    "scores_sign_flipped": ("scores", lambda q, k, scale: -float(scale) * (q @ k.T)),
    "mask_reversed": ("visible", lambda r, c, causal: _orig_visible(r, c, False) if not causal
                      else np.asarray(c)[None, :] >= np.asarray(r)[:, None]),
    "mask_strict": ("visible", lambda r, c, causal: _orig_visible(r, c, False) if not causal
                    else np.asarray(c)[None, :] < np.asarray(r)[:, None]),
    "mask_ignored": ("visible", lambda r, c, causal: _orig_visible(r, c, False)),
    "stats_no_max_shift": ("softmax_stats", _stats_no_shift),
    "stats_l_counts_masked": ("softmax_stats", _stats_mask_ignored_in_l),
    "stats_exp2_for_exp": ("softmax_stats", _stats_exp2),
    "stats_reversed_v": ("softmax_stats", _stats_reversed_v),
    "stats_max_over_masked": ("softmax_stats", _stats_m_from_all_keys),
    "finalize_lse_without_m": ("finalize", lambda m, l, num: (num / l[:, None], np.log(l))),
    "finalize_lse_sign": ("finalize", lambda m, l, num: (num / l[:, None], m - np.log(l))),
    "finalize_unnormalised": ("finalize", lambda m, l, num: (num, m + np.log(l))),
    "finalize_log2": ("finalize", lambda m, l, num: (num / l[:, None], m + np.log2(l))),
    "gqa_heads_interleaved": ("kv_head_of", lambda h, n_heads, n_kv: h % n_kv),
    "window_left_strict": ("visible_window", lambda r, c, wl, wr: (
        (np.ones((len(r), len(c)), dtype=bool) if wl < 0 else np.asarray(c)[None, :] > np.asarray(r)[:, None] - wl)
        & (np.ones((len(r), len(c)), dtype=bool) if wr < 0 else np.asarray(c)[None, :] <= np.asarray(r)[:, None] + wr))),
    "window_sides_swapped": ("visible_window", lambda r, c, wl, wr: _orig_visible_window(r, c, wr, wl)),
    "gqa_heads_reversed": ("kv_head_of", lambda h, n_heads, n_kv: n_kv - 1 - h // (n_heads // n_kv)),
    "block_mask_transposed": ("visible_block_sparse", lambda r, c, bm, bq, bk, causal: (
        np.asarray(bm).astype(bool)[(np.asarray(c) // bk)[None, :], (np.asarray(r) // bq)[:, None]]
        & ((np.asarray(c)[None, :] <= np.asarray(r)[:, None]) if causal else True))),
    "block_sizes_swapped": ("visible_block_sparse", lambda r, c, bm, bq, bk, causal: _orig_visible_bs(
        r, c, bm, bk, bq, causal) if bq != bk else _orig_visible_bs(r, c, bm, bq, bk, causal)),
    "block_causal_dropped": ("visible_block_sparse", lambda r, c, bm, bq, bk, causal: _orig_visible_bs(
        r, c, bm, bq, bk, False)),
    "block_ragged_rounding_up": ("visible_block_sparse", lambda r, c, bm, bq, bk, causal: _orig_visible_bs(
        np.minimum(np.asarray(r) + 1, len(r) - 1), c, bm, bq, bk, causal) & (np.asarray(c)[None, :] <= np.asarray(r)[:, None] if causal else True)),
    "layout_by_batch": ("layout_index", lambda b, h, nb, nh, nl: 0 if nl == 1 else (b if nl == nh else h)),
    "pages_slot_shifted": ("gather_pages", lambda c, row, L, g: np.array(
        [np.asarray(c)[int(row[j // np.asarray(c).shape[1]]), (j + 1) % np.asarray(c).shape[1], g] for j in range(L)]
    ).reshape(L, np.asarray(c).shape[3])),
    "pages_logical_order": ("gather_pages", lambda c, row, L, g: np.asarray(c)[:, :, g].reshape(-1, np.asarray(c).shape[3])[:L]),
    "pages_head_zero": ("gather_pages", lambda c, row, L, g: _orig_gather(c, row, L, 0)),
    "decode_causal_from_start": ("visible_decode", lambda n, L: np.arange(L)[None, :] <= np.arange(n)[:, None]),
    "decode_sees_all_keys": ("visible_decode", lambda n, L: np.ones((n, L), dtype=bool)),
    "decode_excludes_own_key": ("visible_decode", lambda n, L: np.arange(L)[None, :] < (L - n + np.arange(n))[:, None]),
    "window_driver_sides_swapped": ("attention_ref_window", lambda q, k, v, scale, wl, wr: _orig_ref_window(
        q, k, v, scale, wr, wl)),
    "window_driver_heads_ungrouped": ("attention_ref_window", _window_driver_heads(lambda h, n_h, n_kv: h)),
    "window_driver_heads_interleaved": ("attention_ref_window", _window_driver_heads(lambda h, n_h, n_kv: h % n_kv)),
    "window_driver_heads_clamped": ("attention_ref_window", _window_driver_heads(lambda h, n_h, n_kv: min(h, n_kv - 1))),
    "window_probabilities_sum_over_all_keys": ("probabilities_window", _probs_window_all_keys),
    "window_probabilities_over_queries": ("probabilities_window", _probs_window_columns),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
