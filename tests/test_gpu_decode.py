"""GPU parity of decoding from a paged key/value cache (fa2_decode_paged)
against the fp64 oracle, every element, at the forward bars (bf16 inputs:
|O| <= 1e-2, |LSE| <= 1e-3 with fp32 O; a bf16 O may add half an ulp of the
reference).  Tokens that see no key must give exactly O = 0, LSE = -inf.

Caches are seeded with randomly permuted physical pages; context lengths
are ragged (0, 1, below n_q, one key past a page or tile edge, several
chunks), with 1 to 4 new tokens, grouped heads from MHA to MQA, page sizes
of 64 to 256 keys, chunk sizes from one key tile up, d = 64 and 128, and
the largest group (256 query rows per key/value head).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_33_amd as fa2
import oracle.exact_attention as ref
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _bf16_half_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


CASES = [
    # B, H, H_kv, n_q, d, page_size, context_lens, split_keys, o_bf16
    (3, 8, 2, 1, 128, 64, [1, 700, 4096], 0, False),
    (2, 4, 4, 1, 64, 128, [63, 65], 64, False),
    (4, 16, 2, 4, 128, 64, [4, 3, 1000, 257], 256, False),
    (1, 16, 1, 1, 128, 256, [5000], 0, False),
    (2, 8, 8, 2, 128, 64, [0, 130], 128, True),
    (1, 64, 1, 4, 64, 64, [300], 64, False),
    (2, 8, 1, 3, 128, 128, [129, 2], 0, True),
    # chunks of more than 64 pages: the page numbers are read 64 at a time
    (2, 8, 2, 1, 128, 64, [6000, 8191], 8192, False),
    (1, 4, 1, 2, 64, 64, [9000], 4160, False),
    # groups of more than 32 rows: two, four and two (the second of one row)
    # 32-row blocks per group
    (2, 32, 2, 4, 128, 64, [700, 3000], 0, False),
    (1, 16, 1, 8, 64, 64, [1500], 256, True),
    (2, 33, 1, 1, 128, 128, [900, 64], 0, False),
    # many key/value heads: 32 of one row, 16 of two rows, 6 of two rows
    (1, 32, 32, 1, 128, 64, [100], 0, False),
    (2, 16, 16, 2, 64, 128, [300, 77], 64, True),
    (2, 12, 6, 1, 128, 64, [129, 1000], 0, False),
]


@pytest.mark.parametrize("B,H,H_kv,n_q,d,page,lens,split,o_bf16", CASES,
                         ids=[f"{b}x{h}/{hk}-nq{n}-d{d}-p{p}-L{'_'.join(map(str, ls))}-s{s}{'-bf16o' if ob else ''}"
                              for b, h, hk, n, d, p, ls, s, ob in CASES])
def test_decode_every_element(B, H, H_kv, n_q, d, page, lens, split, o_bf16):
    print(f"[case] decode B={B} H={H}/{H_kv} n_q={n_q} d={d} page={page} lens={lens} split={split}", flush=True)
    seed = 1500 + sum(lens) + H
    kc, vc, table = workloads.make_paged_cache(lens, H_kv, d, page, seed)
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn((B, H, n_q, d), generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    ctx = torch.tensor(lens, dtype=torch.int32)
    o_dtype = torch.bfloat16 if o_bf16 else torch.float32
    o, lse = fa2.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), ctx.to(DEV),
                              max_context=max(max(lens), 1), scale=scale, o_dtype=o_dtype, split_keys=split)
    torch.cuda.synchronize()
    eo, el = ref.decode_paged_ref(_np64(q), _np64(kc), _np64(vc), table.numpy(), lens, scale)
    o, lse = _np64(o), _np64(lse)
    empty = np.isneginf(el)
    assert np.array_equal(np.isneginf(lse), empty), "-inf LSE rows differ from the oracle's empty rows"
    assert np.all(o[empty] == 0.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[~empty]))
    err_o = np.abs(o - eo)
    err_l = float(np.max(np.abs(lse[~empty] - el[~empty]))) if (~empty).any() else 0.0
    print(f"[decode] empty rows {int(empty.sum())}, max|dO|={float(np.max(err_o)):.3e} max|dLSE|={err_l:.3e}",
          flush=True)
    assert np.all(err_o <= 1e-2 + (_bf16_half_ulp(eo) if o_bf16 else 0.0))
    assert err_l <= 1e-3


def test_decode_matches_dense_causal_rows():
    """The new tokens' rows equal the last rows of the dense causal kernel on
    the same keys laid out contiguously (two different pipelines)."""
    L, H, d, n_q = 1000, 4, 128, 3
    print("[case] decode vs dense causal forward, L=1000", flush=True)
    kc, vc, table = workloads.make_paged_cache([L], H, d, 64, seed=77)
    pages = table[0, :-(-L // 64)].long()
    k = kc[pages].reshape(-1, H, d)[:L].permute(1, 0, 2).unsqueeze(0).contiguous()
    v = vc[pages].reshape(-1, H, d)[:L].permute(1, 0, 2).unsqueeze(0).contiguous()
    g = torch.Generator().manual_seed(78)
    qfull = torch.randn((1, H, L, d), generator=g).to(torch.bfloat16)
    o1, l1 = fa2.forward(qfull.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    q = qfull[:, :, L - n_q:].contiguous()
    o2, l2 = fa2.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV),
                              torch.tensor([L], dtype=torch.int32, device=DEV), max_context=L, split_keys=256)
    torch.cuda.synchronize()
    d_o = float((o1[:, :, L - n_q:] - o2).abs().max())
    d_l = float((l1[:, :, L - n_q:] - l2).abs().max())
    print(f"[decode] vs dense: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
    assert d_o <= 4e-3 and d_l <= 1e-4


def test_decode_rejections_on_gpu():
    kc, vc, table = workloads.make_paged_cache([100], 2, 128, 64, seed=79)
    q = torch.randn((1, 4, 1, 128)).to(torch.bfloat16).to(DEV)
    ctx = torch.tensor([100], dtype=torch.int32, device=DEV)
    kd, vd, td = kc.to(DEV), vc.to(DEV), table.to(DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        fa2.decode_paged(q, kd, vd, td, ctx, max_context=100, workspace=small)
    kc32, vc32, t32 = workloads.make_paged_cache([100], 2, 128, 32, seed=80)
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.decode_paged(q, kc32.to(DEV), vc32.to(DEV), t32.to(DEV), ctx, max_context=100)
    assert e.value.status == fa2.FA2_ERR_UNSUPPORTED
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.decode_paged(torch.randn((1, 4, 130, 128)).to(torch.bfloat16).to(DEV), kd, vd, td, ctx, max_context=100)
    assert e.value.status == fa2.FA2_ERR_UNSUPPORTED  # 2 x 130 query rows per key/value head


def test_decode_benchmark_batch_sampled_heads():
    """The serving batch the benchmark times (64 sequences, seeded context
    lengths in [1024, 8192], 32 query heads on 8 key/value heads, 64-key
    pages in a permuted cache, the library's chunk size): six (sequence,
    head) pairs against the oracle's page-table gather and causal mask."""
    g = torch.Generator().manual_seed(0)
    B, H, Hkv, d, page = 64, 32, 8, 128, 64
    lens = torch.randint(1024, 8193, (B,), generator=g).tolist()
    kc, vc, table = workloads.make_paged_cache(lens, Hkv, d, page, seed=1)
    q = torch.randn((B, H, 1, d), generator=g).to(torch.bfloat16)
    print(f"[case] decode benchmark batch: {B} sequences, {sum(lens)} keys", flush=True)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa2.decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV),
                              torch.tensor(lens, dtype=torch.int32, device=DEV), max_context=max(lens), scale=scale)
    torch.cuda.synchronize()
    K, V, T = _np64(kc), _np64(vc), table.numpy()
    for b, h in ((0, 0), (63, 31), (17, 5), (40, 12), (5, 30), (33, 3)):
        L = lens[b]
        kv = ref.kv_head_of(h, H, Hkv)
        kb = ref.gather_pages(K, T[b], L, kv)
        vb = ref.gather_pages(V, T[b], L, kv)
        m, l, num = ref.softmax_stats(ref.scores(_np64(q[b, h]), kb, scale), ref.visible_decode(1, L), vb)
        eo, el = ref.finalize(m, l, num)
        err_o = float(np.max(np.abs(_np64(o[b, h]) - eo)))
        err_l = float(np.max(np.abs(_np64(lse[b, h]) - el)))
        print(f"[decode] ({b},{h}) L={L}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
        assert err_o <= 1e-2 and err_l <= 1e-3
