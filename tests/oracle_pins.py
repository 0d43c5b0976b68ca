"""Pins of the fp64 oracle against facts other than the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix.  They are collected in ``PINS`` so
that ``test_oracle.py`` runs them as tests and ``test_oracle_mutants.py`` can
show that a planted mistake anywhere in the oracle makes at least one fail.

All pins look the oracle up through the module object at call time, so a
monkeypatched step function is seen.
"""

from __future__ import annotations

import json
import math
from fractions import Fraction
from pathlib import Path

import numpy as np

import oracle.exact_attention as ref

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _brute_force(q, k, v, scale, causal):
    """The definition with explicit Python loops, math.exp and math.fsum."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        keys = [j for j in range(n) if (not causal) or j <= i]
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(w.values())
        for c in range(dv):
            o[i][c] = math.fsum(w[j] * v[j][c] for j in keys) / den
        lse[i] = mx + math.log(den)
    return np.array(o), np.array(lse)


def pin_brute_force():
    """Tiny random inputs: oracle == explicit loops (N <= 5, d <= 4)."""
    rng = _rng(1234)
    for trial in range(40):
        n = int(rng.integers(1, 6))
        d = int(rng.integers(1, 5))
        dv = int(rng.integers(1, 5))
        q, k = rng.normal(size=(n, d)), rng.normal(size=(n, d))
        v = rng.normal(size=(n, dv))
        scale = float(rng.choice([0.1, 0.5, 1.0, 2.7]))
        for causal in (False, True):
            eo, el = _brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal)
            o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], scale, causal)
            _close(o[0, 0], eo, 1e-12, f"brute O trial {trial} causal={causal}")
            _close(lse[0, 0], el, 1e-12, f"brute LSE trial {trial} causal={causal}")


def _parse_scale(spec):
    if isinstance(spec, dict) and "ln" in spec:
        return math.log(float(Fraction(spec["ln"])))
    return float(spec)


def pin_hand_cases():
    """Hand-derived rational outputs (tests/golden/hand_cases.json)."""
    data = json.loads((GOLDEN / "hand_cases.json").read_text())
    for case in data["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        v = np.array(case["v"], dtype=np.float64)
        scale = _parse_scale(case["scale"])
        eo = np.vectorize(lambda s: float(Fraction(s)))(np.array(case["o"], dtype=object)).astype(np.float64)
        el = np.vectorize(lambda s: math.log(float(Fraction(s))))(np.array(case["lse_ln_of"], dtype=object)).astype(np.float64)
        o, lse = ref.attention_ref(q, k, v, scale, case["causal"])
        _close(o, eo, 1e-12, f"hand case {case['name']} O")
        _close(lse, el, 1e-12, f"hand case {case['name']} LSE")


def pin_probability_rows():
    """With V = I the output rows are the probability rows: >= 0, sum to 1,
    zero above the diagonal when causal, and the LSE normalises them."""
    rng = _rng(7)
    n, d = 9, 5
    q, k = rng.normal(size=(n, d)), rng.normal(size=(n, d))
    eye = np.eye(n)
    scale = 0.7
    for causal in (False, True):
        p, lse = ref.attention_ref(q[None, None], k[None, None], eye[None, None], scale, causal)
        p, lse = p[0, 0], lse[0, 0]
        assert np.all(p >= 0.0), "negative probability"
        _close(p.sum(axis=1), np.ones(n), 1e-13, f"row sums causal={causal}")
        if causal:
            assert np.all(np.triu(p, 1) == 0.0), "causal mass above the diagonal"
        # p_ij = exp(S_ij - LSE_i) for visible keys
        s = scale * (q @ k.T)
        vis = np.tril(np.ones((n, n), dtype=bool)) if causal else np.ones((n, n), dtype=bool)
        _close(np.where(vis, p, 0.0), np.where(vis, np.exp(s - lse[:, None]), 0.0), 1e-13,
               f"p = exp(S - LSE) causal={causal}")


def pin_constant_v():
    """If every value row is the same vector c, every output row is c."""
    rng = _rng(11)
    n, d = 17, 6
    q, k = rng.normal(size=(n, d)) * 3, rng.normal(size=(n, d)) * 3
    c = rng.normal(size=(4,))
    v = np.tile(c, (n, 1))
    for causal in (False, True):
        o, _ = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.9, causal)
        _close(o[0, 0], np.tile(c, (n, 1)), 1e-13, f"constant V causal={causal}")


def pin_kv_permutation():
    """Non-causal attention ignores the order of the key/value pairs."""
    rng = _rng(13)
    n, d = 23, 8
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 3))
    perm = rng.permutation(n)
    o1, l1 = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.4, False)
    o2, l2 = ref.attention_ref(q[None, None], k[perm][None, None], v[perm][None, None], 0.4, False)
    _close(o1, o2, 1e-13, "permuted O")
    _close(l1, l2, 1e-13, "permuted LSE")


def pin_merge_identity():
    """Statistics of disjoint key chunks merge into the full result
    (Mishra: running max, denominator and numerator are mergeable)."""
    rng = _rng(17)
    n, d = 31, 6
    q, k, v = rng.normal(size=(n, d)) * 2, rng.normal(size=(n, d)) * 2, rng.normal(size=(n, 5))
    for causal in (False, True):
        o_ref, l_ref = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.8, causal)
        for n_chunks in (2, 3, 4):
            ids = rng.permutation(n)
            parts = [ref.partial_stats(q, k, v, 0.8, causal, c) for c in np.array_split(ids, n_chunks)]
            m, l, num = ref.merge_stats(parts)
            o, lse = ref.finalize(m, l, num)
            _close(o, o_ref[0, 0], 1e-12, f"merged O ({n_chunks} chunks, causal={causal})")
            _close(lse, l_ref[0, 0], 1e-12, f"merged LSE ({n_chunks} chunks, causal={causal})")
            # LSE of the union is log-sum-exp of the chunk LSEs
            chunk_lse = []
            for m_a, l_a, _ in parts:
                with np.errstate(divide="ignore"):
                    chunk_lse.append(np.where(l_a > 0, m_a + np.log(np.where(l_a > 0, l_a, 1.0)), -np.inf))
            top = np.max(chunk_lse, axis=0)
            _close(top + np.log(np.sum(np.exp(np.array(chunk_lse) - top), axis=0)), l_ref[0, 0], 1e-12,
                   "LSE of union")


def pin_tiled_schedules():
    """The pages' tiled online softmax -- with the division deferred (FA2) or
    done every step (FA1) -- lands on the oracle's output (Saraf 2.2, 3);
    normalisation counts are T_q versus T_q*T_k."""
    rng = _rng(19)
    n, d = 150, 8
    q, k, v = rng.normal(size=(n, d)) * 2, rng.normal(size=(n, d)) * 2, rng.normal(size=(n, 4))
    for causal in (False, True):
        o_ref, l_ref = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.6, causal)
        for br, bc in ((64, 64), (32, 48), (7, 5)):
            o2, l2, n2 = ref.tiled_online_attention(q, k, v, 0.6, causal, br, bc, normalize_each_step=False)
            o1, l1, _ = ref.tiled_online_attention(q, k, v, 0.6, causal, br, bc, normalize_each_step=True)
            _close(o2, o_ref[0, 0], 1e-12, f"deferred division O br={br} bc={bc} causal={causal}")
            _close(l2, l_ref[0, 0], 1e-12, f"deferred division LSE br={br} bc={bc}")
            _close(o1, o_ref[0, 0], 1e-12, f"per-step normalisation O br={br} bc={bc} causal={causal}")
            _close(l1, l_ref[0, 0], 1e-12, f"per-step normalisation LSE br={br} bc={bc}")
            assert n2 == -(-n // br), "deferred schedule divides once per query block"
    # Saraf 2.2: at 8192 tokens, 64-row blocks: 16,384 per-step rescales vs 128 divisions.
    n = 8192
    qs = rng.normal(size=(n, 2))
    _, _, n_fa1 = ref.tiled_online_attention(qs, qs, qs[:, :1], 0.1, False, 64, 64, normalize_each_step=True)
    _, _, n_fa2 = ref.tiled_online_attention(qs, qs, qs[:, :1], 0.1, False, 64, 64, normalize_each_step=False)
    assert (n_fa1, n_fa2) == (16384, 128), (n_fa1, n_fa2)


def pin_scale_zero():
    """scale = 0: uniform weights over visible keys; LSE = ln(#visible)."""
    rng = _rng(23)
    n, d = 12, 4
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 3))
    o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.0, False)
    _close(o[0, 0], np.tile(v.mean(axis=0), (n, 1)), 1e-13, "scale=0 O")
    _close(lse[0, 0], np.full(n, math.log(n)), 1e-13, "scale=0 LSE")
    o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.0, True)
    _close(o[0, 0], np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None], 1e-13, "scale=0 causal O")
    _close(lse[0, 0], np.log(np.arange(1, n + 1)), 1e-13, "scale=0 causal LSE")


def pin_single_key_rows():
    """Causal row 0 sees only key 0; N = 1 sees only itself: O = v, LSE = scale q.k."""
    rng = _rng(29)
    n, d = 6, 5
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 3))
    o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], 1.3, True)
    _close(o[0, 0, 0], v[0], 1e-14, "causal row 0 O")
    _close(lse[0, 0, 0], 1.3 * float(q[0] @ k[0]), 1e-13, "causal row 0 LSE")
    for causal in (False, True):
        o, lse = ref.attention_ref(q[None, None, :1], k[None, None, :1], v[None, None, :1], 1.3, causal)
        _close(o[0, 0], v[:1], 1e-14, "N=1 O")
        _close(lse[0, 0], [1.3 * float(q[0] @ k[0])], 1e-13, "N=1 LSE")


def pin_key_shift():
    """k_j -> k_j + u for all j: O unchanged, LSE_i shifts by scale * q_i.u."""
    rng = _rng(31)
    n, d = 19, 6
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 4))
    u = rng.normal(size=(d,))
    for causal in (False, True):
        o1, l1 = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.5, causal)
        o2, l2 = ref.attention_ref(q[None, None], (k + u)[None, None], v[None, None], 0.5, causal)
        _close(o2, o1, 1e-12, f"key shift O causal={causal}")
        _close(l2[0, 0], l1[0, 0] + 0.5 * (q @ u), 1e-12, f"key shift LSE causal={causal}")


def pin_causal_prefix():
    """Causal rows [0, M) do not depend on keys >= M; causal row i equals
    non-causal attention over keys 0..i."""
    rng = _rng(37)
    n, d = 21, 5
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 3))
    o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.7, True)
    for m in (1, 8, 13):
        op, lp = ref.attention_ref(q[None, None, :m], k[None, None, :m], v[None, None, :m], 0.7, True)
        _close(o[0, 0, :m], op[0, 0], 1e-13, f"prefix {m} O")
        _close(lse[0, 0, :m], lp[0, 0], 1e-13, f"prefix {m} LSE")
    for i in (0, 5, 20):
        s = 0.7 * (k[:i + 1] @ q[i])
        w = np.exp(s - s.max())
        _close(o[0, 0, i], (w @ v[:i + 1]) / w.sum(), 1e-13, f"causal row {i} as non-causal prefix")
        _close(lse[0, 0, i], s.max() + math.log(w.sum()), 1e-13, f"causal row {i} LSE")


def pin_large_scores():
    """Huge, well-separated scores (exp would overflow without the max
    shift): the softmax is one-hot on the argmax, LSE = its score."""
    rng = _rng(41)
    n, d = 10, 3
    q = rng.normal(size=(n, d))
    k = rng.normal(size=(n, d))
    v = rng.normal(size=(n, 2))
    s = q @ k.T
    srt = np.sort(s, axis=1)
    assert np.all(srt[:, -1] - srt[:, -2] > 1e-3)
    scale = 2.0e6
    o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], scale, False)
    arg = np.argmax(s, axis=1)
    _close(o[0, 0], v[arg], 1e-12, "one-hot O")
    _close(lse[0, 0] / scale, s.max(axis=1), 1e-9, "LSE / scale = max score")
    # causal: one-hot on the argmax over keys 0..i only (hidden keys may score higher)
    s_c = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    srt = np.sort(s_c, axis=1)
    sep = np.where(np.isfinite(srt[:, -2]), srt[:, -1] - srt[:, -2], np.inf)
    assert np.all(sep > 1e-3)
    assert np.any(s.max(axis=1) - s_c.max(axis=1) > 1.0), "want hidden keys that outscore visible ones"
    o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], scale, True)
    _close(o[0, 0], v[np.argmax(s_c, axis=1)], 1e-12, "causal one-hot O")
    _close(lse[0, 0] / scale, s_c.max(axis=1), 1e-9, "causal LSE / scale = max visible score")


def pin_rows_helper():
    """attention_rows for selected rows == the same rows of the full result."""
    rng = _rng(43)
    n, d = 40, 6
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 6))
    rows = np.array([0, 1, 17, 38, 39])
    for causal in (False, True):
        o, lse = ref.attention_ref(q[None, None], k[None, None], v[None, None], 0.3, causal)
        orow, lrow = ref.attention_rows(q, k, v, 0.3, causal, rows)
        _close(orow, o[0, 0, rows], 1e-14, "rows helper O")
        _close(lrow, lse[0, 0, rows], 1e-14, "rows helper LSE")


def pin_batch_heads():
    """[B, H, N, d] inputs are independent per (b, h)."""
    rng = _rng(47)
    B, H, n, d = 2, 3, 7, 4
    q, k, v = rng.normal(size=(B, H, n, d)), rng.normal(size=(B, H, n, d)), rng.normal(size=(B, H, n, d))
    o, lse = ref.attention_ref(q, k, v, 0.5, True)
    for b in range(B):
        for h in range(H):
            eo, el = _brute_force(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.5, True)
            _close(o[b, h], eo, 1e-12, f"batch/head ({b},{h}) O")
            _close(lse[b, h], el, 1e-12, f"batch/head ({b},{h}) LSE")


def pin_gqa_head_groups():
    """Grouped key/value heads: with 6 query heads on 3 key/value heads the
    query heads read key/value heads 0, 0, 1, 1, 2, 2; on 1 they all read 0;
    on 6 the result is ordinary multi-head attention.  Each query head is
    checked against the one-head oracle on the key/value head it must use."""
    rng = _rng(21)
    n, d = 13, 4
    q = rng.normal(size=(1, 6, n, d))
    for hkv, expect in ((3, [0, 0, 1, 1, 2, 2]), (1, [0] * 6), (6, list(range(6)))):
        k, v = rng.normal(size=(1, hkv, n, d)), rng.normal(size=(1, hkv, n, d))
        for causal in (False, True):
            o, lse = ref.attention_ref_gqa(q, k, v, 0.6, causal)
            for h, g in enumerate(expect):
                eo, el = ref.attention_head(q[0, h], k[0, g], v[0, g], 0.6, causal)
                _close(o[0, h], eo, 1e-14, f"GQA H_kv={hkv} head {h} O causal={causal}")
                _close(lse[0, h], el, 1e-14, f"GQA H_kv={hkv} head {h} LSE causal={causal}")
    try:
        ref.attention_ref_gqa(q, rng.normal(size=(1, 4, n, d)), rng.normal(size=(1, 4, n, d)), 0.6, False)
    except ValueError:
        pass
    else:
        raise AssertionError("6 query heads on 4 key/value heads must be rejected")


def _brute_force_window(q, k, v, scale, wl, wr):
    """Sliding-window attention by explicit loops: the keys of row i are
    those j with i - wl <= j (if wl >= 0) and j <= i + wr (if wr >= 0)."""
    n, d, dv = len(q), len(q[0]), len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        keys = [j for j in range(len(k)) if (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)]
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(w.values())
        for c in range(dv):
            o[i][c] = math.fsum(w[j] * v[j][c] for j in keys) / den
        lse[i] = mx + math.log(den)
    return np.array(o), np.array(lse)


def pin_window_brute_force():
    """Sliding windows on tiny random heads: oracle == explicit loops."""
    rng = _rng(31)
    for trial in range(8):
        n = int(rng.integers(1, 9))
        q, k, v = rng.normal(size=(n, 3)), rng.normal(size=(n, 3)), rng.normal(size=(n, 2))
        for wl, wr in ((0, 0), (1, 0), (2, 3), (-1, 2), (3, -1), (-1, 0), (-1, -1), (0, 2)):
            eo, el = _brute_force_window(q.tolist(), k.tolist(), v.tolist(), 0.8, wl, wr)
            o, lse = ref.attention_head_window(q, k, v, 0.8, wl, wr)
            _close(o, eo, 1e-12, f"window ({wl},{wr}) O trial {trial}")
            _close(lse, el, 1e-12, f"window ({wl},{wr}) LSE trial {trial}")


def pin_window_special_cases():
    """Window (0, 0): each row sees only its own key, so O_i = v_i and
    LSE_i = S_ii.  Window (-1, 0) is the causal mask; (-1, -1) and windows
    of at least N keys on both sides are no mask at all."""
    rng = _rng(32)
    n, d = 11, 5
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 3))
    o, lse = ref.attention_head_window(q, k, v, 0.6, 0, 0)
    _close(o, v, 1e-14, "window (0,0) O = V")
    _close(lse, 0.6 * np.einsum("id,id->i", q, k), 1e-13, "window (0,0) LSE = S_ii")
    oc, lc = ref.attention_head(q, k, v, 0.6, True)
    for wl, wr, (eo, el) in ((-1, 0, (oc, lc)), (n, 0, (oc, lc))):
        o, lse = ref.attention_head_window(q, k, v, 0.6, wl, wr)
        _close(o, eo, 1e-14, f"window ({wl},{wr}) vs causal O")
        _close(lse, el, 1e-14, f"window ({wl},{wr}) vs causal LSE")
    of, lf = ref.attention_head(q, k, v, 0.6, False)
    for wl, wr in ((-1, -1), (n, n), (-1, n)):
        o, lse = ref.attention_head_window(q, k, v, 0.6, wl, wr)
        _close(o, of, 1e-14, f"window ({wl},{wr}) vs full O")
        _close(lse, lf, 1e-14, f"window ({wl},{wr}) vs full LSE")


def pin_window_probabilities():
    """probabilities_window (the probabilities the window gradients are built
    from) on tiny random heads: each row equals exp(s_ij) / sum over the row's
    band by explicit loops, is zero outside the band and sums to 1; the
    window (-1, 0) gives the causal probabilities."""
    rng = _rng(37)
    for n, d, wl, wr in ((5, 3, 1, 1), (6, 2, -1, 2), (7, 4, 2, -1), (4, 2, 0, 0), (6, 3, 3, 1)):
        q = rng.standard_normal((n, d))
        k = rng.standard_normal((n, d))
        scale = 0.7
        p = ref.probabilities_window(q, k, scale, wl, wr)
        for i in range(n):
            band = [j for j in range(n) if (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)]
            s = {j: scale * math.fsum(q[i, t] * k[j, t] for t in range(d)) for j in band}
            den = math.fsum(math.exp(x) for x in s.values())
            for j in range(n):
                want = math.exp(s[j]) / den if j in s else 0.0
                assert abs(p[i, j] - want) <= 1e-12, (n, wl, wr, i, j, p[i, j], want)
            assert abs(math.fsum(p[i]) - 1.0) <= 1e-12
    q = rng.standard_normal((9, 4))
    k = rng.standard_normal((9, 4))
    assert np.allclose(ref.probabilities_window(q, k, 0.5, -1, 0), ref.probabilities(q, k, 0.5, True),
                       rtol=0, atol=1e-14)


def pin_window_driver_grouped_heads():
    """The [B, H] sliding-window driver: 6 query heads on 3 key/value heads
    (query head h reads key/value head 0, 0, 1, 1, 2, 2) and on 1, two
    sequences, windows that differ on the two sides.  Every (b, h) must equal
    the loop-evaluated window attention on the key/value head it reads."""
    rng = _rng(33)
    B, H, n, d = 2, 6, 6, 3
    q = rng.normal(size=(B, H, n, d))
    for hkv, groups in ((3, [0, 0, 1, 1, 2, 2]), (1, [0] * 6)):
        k, v = rng.normal(size=(B, hkv, n, d)), rng.normal(size=(B, hkv, n, 2))
        for wl, wr in ((2, 0), (1, 3), (-1, 2), (3, -1)):
            o, lse = ref.attention_ref_window(q, k, v, 0.7, wl, wr)
            assert o.shape == (B, H, n, 2) and lse.shape == (B, H, n)
            for b in range(B):
                for h in range(H):
                    g = groups[h]
                    eo, el = _brute_force_window(q[b, h].tolist(), k[b, g].tolist(), v[b, g].tolist(), 0.7, wl, wr)
                    tag = f"window driver H_kv={hkv} ({wl},{wr}) (b,h)=({b},{h})"
                    _close(o[b, h], eo, 1e-12, tag + " O")
                    _close(lse[b, h], el, 1e-12, tag + " LSE")


def _same_with_inf(a, b, tol, what):
    """Equal -inf entries, the rest within tol."""
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    ia, ib = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(ia, ib), f"{what}: -inf at different places"
    _close(a[~ia], b[~ib], tol, what)


def _brute_force_block_sparse(q, k, v, scale, bm, bq, bk, causal):
    """Block-sparse attention by explicit loops: the keys of row i are the j
    whose block (i // bq, j // bk) is set (and j <= i when causal); a row
    with no key gets O = 0 and LSE = -inf."""
    n, d, dv = len(q), len(q[0]), len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [-math.inf] * n
    for i in range(n):
        keys = [j for j in range(len(k)) if bm[i // bq][j // bk] and (not causal or j <= i)]
        if not keys:
            continue
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(w.values())
        for c in range(dv):
            o[i][c] = math.fsum(w[j] * v[j][c] for j in keys) / den
        lse[i] = mx + math.log(den)
    return np.array(o), np.array(lse)


def pin_block_sparse_brute_force():
    """Random block masks (non-square blocks, ragged last blocks, empty rows)
    on tiny heads: oracle == explicit loops."""
    rng = _rng(41)
    for trial in range(12):
        n = int(rng.integers(1, 10))
        bq, bk = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        bm = rng.random(size=(-(-n // bq), -(-n // bk))) < 0.5
        q, k, v = rng.normal(size=(n, 3)), rng.normal(size=(n, 3)), rng.normal(size=(n, 2))
        for causal in (False, True):
            eo, el = _brute_force_block_sparse(q.tolist(), k.tolist(), v.tolist(), 0.7, bm.tolist(), bq, bk, causal)
            o, lse = ref.attention_head_block_sparse(q, k, v, 0.7, bm, bq, bk, causal)
            _close(o, eo, 1e-12, f"block-sparse O trial {trial} causal={causal}")
            _same_with_inf(lse, el, 1e-12, f"block-sparse LSE trial {trial} causal={causal}")


def pin_block_sparse_special_cases():
    """An all-ones mask is dense attention; a block-diagonal mask of b-row
    blocks is dense attention on each b-row chunk on its own; an all-zero
    mask gives O = 0 and LSE = -inf everywhere."""
    rng = _rng(42)
    n, d = 14, 4
    q, k, v = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, 3))
    for causal in (False, True):
        eo, el = ref.attention_head(q, k, v, 0.5, causal)
        o, lse = ref.attention_head_block_sparse(q, k, v, 0.5, np.ones((5, 3), dtype=bool), 3, 5, causal)
        _close(o, eo, 1e-14, f"all-ones mask O causal={causal}")
        _close(lse, el, 1e-14, f"all-ones mask LSE causal={causal}")
        b = 4
        diag = np.eye(-(-n // b), dtype=bool)
        o, lse = ref.attention_head_block_sparse(q, k, v, 0.5, diag, b, b, causal)
        for c0 in range(0, n, b):
            sl = slice(c0, min(n, c0 + b))
            eo, el = ref.attention_head(q[sl], k[sl], v[sl], 0.5, causal)
            _close(o[sl], eo, 1e-14, f"block-diagonal O rows {c0}.. causal={causal}")
            _close(lse[sl], el, 1e-14, f"block-diagonal LSE rows {c0}.. causal={causal}")
    o, lse = ref.attention_head_block_sparse(q, k, v, 0.5, np.zeros((2, 2), dtype=bool), 7, 7, False)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def pin_block_sparse_layouts():
    """One mask for all heads, one per head, or one per (sequence, head):
    each (b, h) uses the mask its index names."""
    rng = _rng(43)
    B, H, n = 2, 3, 6
    q, k, v = rng.normal(size=(B, H, n, 3)), rng.normal(size=(B, H, n, 3)), rng.normal(size=(B, H, n, 2))
    masks = rng.random(size=(B * H, 3, 2)) < 0.6
    masks[:, :, 0] = True  # keep every row non-empty
    for L in (1, H, B * H):
        o, lse = ref.attention_ref_block_sparse(q, k, v, 0.9, masks[:L], 2, 3, False)
        for b in range(B):
            for h in range(H):
                idx = {1: 0, H: h, B * H: b * H + h}[L]
                eo, el = _brute_force_block_sparse(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.9,
                                                   masks[idx].tolist(), 2, 3, False)
                _close(o[b, h], eo, 1e-12, f"layouts L={L} O ({b},{h})")
                _close(lse[b, h], el, 1e-12, f"layouts L={L} LSE ({b},{h})")
    try:
        ref.attention_ref_block_sparse(q, k, v, 0.9, masks[:4], 2, 3, False)
    except ValueError:
        pass
    else:
        raise AssertionError("4 masks for B=2, H=3 must be rejected")


def _paged_cache(rng, kv, page_size, n_pages_total):
    """Scatter per-sequence contiguous keys kv[b] ([L_b, H_kv, d]) into a
    paged cache with randomly permuted physical pages; returns (cache, table)."""
    perm = rng.permutation(n_pages_total)
    Hkv, d = kv[0].shape[1], kv[0].shape[2]
    max_pages = max(-(-len(x) // page_size) for x in kv) or 1
    cache = rng.normal(size=(n_pages_total, page_size, Hkv, d))  # unused slots hold noise
    table = np.full((len(kv), max_pages), -1, dtype=np.int64)
    nxt = 0
    for b, x in enumerate(kv):
        for p in range(-(-len(x) // page_size)):
            phys = perm[nxt]
            nxt += 1
            table[b, p] = phys
            chunk = x[p * page_size:(p + 1) * page_size]
            cache[phys, :len(chunk)] = chunk
    return cache, table


def pin_decode_matches_causal_rows():
    """Paged decoding of the n_q newest tokens equals the last n_q rows of
    plain causal attention over the same keys laid out contiguously,
    whatever the physical page order."""
    rng = _rng(51)
    for trial in range(4):
        B, Hkv, G, d, page = 2, 2, 2, 5, int(rng.integers(2, 5))
        n_q = int(rng.integers(1, 4))
        lens = [int(rng.integers(n_q, 17)) for _ in range(B)]
        ks = [rng.normal(size=(L, Hkv, d)) for L in lens]
        vs = [rng.normal(size=(L, Hkv, d)) for L in lens]
        n_pages = sum(-(-L // page) for L in lens) + 3
        kc, table = _paged_cache(np.random.default_rng(trial), ks, page, n_pages)
        vc, table_v = _paged_cache(np.random.default_rng(trial), vs, page, n_pages)
        assert np.array_equal(table, table_v)
        q = rng.normal(size=(B, Hkv * G, n_q, d))
        o, lse = ref.decode_paged_ref(q, kc, vc, table, lens, 0.6)
        for b in range(B):
            L = lens[b]
            for h in range(Hkv * G):
                g = h // G
                qfull = rng.normal(size=(L, d))
                qfull[L - n_q:] = q[b, h]
                eo, el = ref.attention_rows(qfull, ks[b][:, g], vs[b][:, g], 0.6, True, np.arange(L - n_q, L))
                _close(o[b, h], eo, 1e-12, f"decode O trial {trial} ({b},{h})")
                _close(lse[b, h], el, 1e-12, f"decode LSE trial {trial} ({b},{h})")


def pin_decode_brute_force():
    """Tiny paged caches by explicit loops and page lookups, including
    tokens whose position is below 0 (no key: O = 0, LSE = -inf)."""
    rng = _rng(52)
    for trial in range(6):
        B, Hkv, G, d, page = 2, 1 + trial % 2, 2, 3, 2 + trial % 2
        n_q = 1 + trial % 3
        lens = [int(rng.integers(0, 9)) for _ in range(B)]
        n_pages = 12
        kc = rng.normal(size=(n_pages, page, Hkv, d))
        vc = rng.normal(size=(n_pages, page, Hkv, 2))
        table = np.stack([rng.permutation(n_pages)[:6] for _ in range(B)])
        q = rng.normal(size=(B, Hkv * G, n_q, d))
        o, lse = ref.decode_paged_ref(q, kc, vc, table, lens, 0.9)
        for b in range(B):
            for h in range(Hkv * G):
                g = h // G
                for i in range(n_q):
                    pos = lens[b] - n_q + i
                    keys = list(range(0, pos + 1)) if pos >= 0 else []
                    if not keys:
                        assert np.all(o[b, h, i] == 0.0) and np.isneginf(lse[b, h, i])
                        continue
                    kk = {j: kc[table[b][j // page], j % page, g] for j in keys}
                    vv = {j: vc[table[b][j // page], j % page, g] for j in keys}
                    s = {j: 0.9 * math.fsum(q[b, h, i, t] * kk[j][t] for t in range(d)) for j in keys}
                    mx = max(s.values())
                    w = {j: math.exp(s[j] - mx) for j in keys}
                    den = math.fsum(w.values())
                    eo = [math.fsum(w[j] * vv[j][c] for j in keys) / den for c in range(2)]
                    _close(o[b, h, i], eo, 1e-12, f"decode brute O trial {trial}")
                    _close(lse[b, h, i], mx + math.log(den), 1e-12, f"decode brute LSE trial {trial}")


PINS = [
    pin_decode_matches_causal_rows,
    pin_decode_brute_force,
    pin_block_sparse_brute_force,
    pin_block_sparse_special_cases,
    pin_block_sparse_layouts,
    pin_window_brute_force,
    pin_window_special_cases,
    pin_window_probabilities,
    pin_window_driver_grouped_heads,
    pin_gqa_head_groups,
    pin_brute_force,
    pin_hand_cases,
    pin_probability_rows,
    pin_constant_v,
    pin_kv_permutation,
    pin_merge_identity,
    pin_tiled_schedules,
    pin_scale_zero,
    pin_single_key_rows,
    pin_key_shift,
    pin_causal_prefix,
    pin_large_scores,
    pin_rows_helper,
    pin_batch_heads,
]
