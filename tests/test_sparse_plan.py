"""Block-sparse key-tile lists on the CPU: fa2_sparse_plan lists exactly the
key tiles in which each 32-row slice of a query tile sees a key (brute force
from the oracle's block-sparse visibility), and the sparse entry points
reject malformed calls before any HIP call.  No compute call is made here.
"""

import numpy as np
import pytest

import exact_tiled_attention_33_amd as fa2
import oracle.exact_attention as ref
import workloads

BR, BC, SL = 256, 64, 32


def _expected(N, bm, bq, bk, causal):
    """Per (layout, tile): list of (key tile, slice bits) from the oracle's mask."""
    out = []
    ids = np.arange(N)
    T, nk = -(-N // BR), -(-N // BC)
    for L in range(bm.shape[0]):
        vis = ref.visible_block_sparse(ids, ids, bm[L], bq, bk, causal)
        for t in range(T):
            lst = []
            for j in range(nk):
                bits = 0
                for s in range(8):
                    r0 = t * BR + s * SL
                    if r0 >= N:
                        break
                    if vis[r0:min(N, r0 + SL), j * BC:min(N, (j + 1) * BC)].any():
                        bits |= 1 << s
                if bits:
                    lst.append((j, bits))
            out.append(lst)
    return out


@pytest.mark.parametrize("N, bq, bk, L, density, causal", [
    (700, 32, 64, 1, 0.4, False), (700, 128, 128, 2, 0.5, True), (1000, 64, 192, 1, 0.3, True),
    (513, 256, 64, 3, 0.6, False), (129, 96, 128, 1, 0.5, True), (2049, 512, 256, 2, 0.25, True),
])
def test_lists_match_oracle_visibility(N, bq, bk, L, density, causal):
    bm = workloads.make_block_mask(L, -(-N // bq), -(-N // bk), density, seed=N + bq, keep_diagonal=False)
    plan = fa2.fa2_sparse_plan(N, bq, bk, bm, causal)
    exp = _expected(N, bm, bq, bk, causal)
    assert plan.tile_ptr[0] == 0 and plan.tile_ptr[-1] == plan.n_entries
    assert np.all(np.diff(plan.tile_ptr) >= 0)
    for idx, lst in enumerate(exp):
        got = plan.entries[plan.tile_ptr[idx]:plan.tile_ptr[idx + 1]]
        assert [(int(e) & 0xFFFFFF, int(e) >> 24) for e in got] == lst, idx


def test_all_ones_mask_lists_every_needed_tile():
    N = 1000
    bm = np.ones((1, -(-N // 128), -(-N // 128)), dtype=bool)
    full = fa2.fa2_sparse_plan(N, 128, 128, bm, False)
    assert full.n_entries == 4 * 16 and np.all(full.entries >> 24 == 0xFF)
    causal = fa2.fa2_sparse_plan(N, 128, 128, bm, True)
    # tile t lists key tiles 0 .. its last row / 64
    assert list(np.diff(causal.tile_ptr)) == [4, 8, 12, 16]


def test_credited_pairs_block_sparse_matches_oracle_mask():
    rng = np.random.default_rng(5)
    for N, bq, bk, causal in ((300, 64, 128, True), (300, 96, 64, False), (77, 32, 64, True)):
        bm = rng.random(size=(-(-N // bq), -(-N // bk))) < 0.5
        ids = np.arange(N)
        exp = int(ref.visible_block_sparse(ids, ids, bm, bq, bk, causal).sum())
        assert workloads.credited_pairs_block_sparse(N, bm, bq, bk, causal) == exp


def test_sparse_plan_validation():
    bm = np.ones((1, 4, 4), dtype=np.uint8)
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.fa2_sparse_plan(1024, 48, 256, np.ones((1, 22, 4)), False)
    assert e.value.status == fa2.FA2_ERR_UNSUPPORTED
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.fa2_sparse_plan(1024, 256, 32, np.ones((1, 4, 32)), False)
    assert e.value.status == fa2.FA2_ERR_UNSUPPORTED
    lib = fa2.load()
    import ctypes
    n = ctypes.c_int(0)
    assert lib.fa2_sparse_plan(1024, 256, 256, 1, None, 0, None, None, 0, ctypes.byref(n)) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_sparse_plan(1024, 256, 256, 1, bm.ctypes.data, 2, None, None, 0, ctypes.byref(n)) == fa2.FA2_ERR_INVALID_ARG
    ptr = np.zeros(5, dtype=np.int32)
    ent = np.zeros(3, dtype=np.uint32)
    st = lib.fa2_sparse_plan(1024, 256, 256, 1, bm.ctypes.data, 0, ptr.ctypes.data, ent.ctypes.data, 3,
                             ctypes.byref(n))
    assert st == fa2.FA2_ERR_INVALID_ARG  # 16 entries do not fit in 3
    with pytest.raises(ValueError):
        fa2.fa2_sparse_plan(1024, 256, 256, np.ones((1, 3, 4)), False)


Q, K, V, O, L, P, E = (0x10000000 * (i + 1) for i in range(7))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Hkv=3, N=1024, d=128, causal=1, scale=0.125, stream=0,
            in_dtype=fa2.BF16, o_dtype=fa2.F32, n_layouts=3, ptr=P, ent=E, n_ent=40)


def _call(**over):
    a = dict(GOOD, **over)
    return fa2.fa2_fwd_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                              a["causal"], a["scale"], a["stream"], a["in_dtype"], a["o_dtype"], a["n_layouts"],
                              a["ptr"], a["ent"], a["n_ent"])


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.parametrize("over, status", [
    (dict(n_layouts=2), fa2.FA2_ERR_INVALID_ARG),
    (dict(n_layouts=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(ptr=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(ptr=P + 2), fa2.FA2_ERR_INVALID_ARG),
    (dict(ent=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(n_ent=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(causal=2), fa2.FA2_ERR_INVALID_ARG),
    (dict(ptr=O), fa2.FA2_ERR_INVALID_ARG),
    (dict(ent=L), fa2.FA2_ERR_INVALID_ARG),
    (dict(in_dtype=fa2.F32), fa2.FA2_ERR_UNSUPPORTED),
    (dict(d=80), fa2.FA2_ERR_UNSUPPORTED),
    (dict(Hkv=2), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa2.FA2_ERR_INVALID_ARG),
])
def test_fwd_sparse_validation(over, status):
    assert _call(**over) == status


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_fwd_sparse_no_device_status_on_cpu_only_host():
    for over in (dict(), dict(n_layouts=1), dict(n_layouts=6), dict(ent=0, n_ent=0), dict(causal=0)):
        assert _call(**over) == fa2.FA2_ERR_NO_DEVICE
