"""fa2_decode_paged_noalloc, the decode entry point that allocates nothing
(partials in the library's static per-device scratch), against
fa2_decode_paged with a caller workspace: the same kernels with the same
chunk size, so o and lse must agree bit for bit.

Two calls in a row share the scratch: the first is the serving batch the
benchmark times (64 sequences, context lengths in [1024, 8192], 32 query
heads on 8 key/value heads), the second a smaller ragged batch that reads
only part of what the first wrote.  A third call needs more than the
scratch and must be refused before any launch.
"""

from __future__ import annotations

import math

import pytest
import torch

import exact_tiled_attention_33_amd as fa2
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _batch(lens, H, H_kv, n_q, d, page, seed):
    kc, vc, table = workloads.make_paged_cache(lens, H_kv, d, page, seed=seed, device=DEV)
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn((len(lens), H, n_q, d), generator=g).to(torch.bfloat16).to(DEV)
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return q, kc, vc, table, ctx


def _both(q, kc, vc, table, ctx, max_ctx, o_dtype, stream):
    B, H, n_q, d = q.shape
    n_pages, page, H_kv, _ = kc.shape
    units = torch.cuda.get_device_properties(DEV).multi_processor_count
    split, ws_bytes = fa2.fa2_decode_paged_workspace(B, H, H_kv, n_q, d, max_ctx, 0, units)
    assert ws_bytes <= fa2.FA2_DECODE_SCRATCH_BYTES
    scale = 1.0 / math.sqrt(d)
    code = fa2.BF16 if o_dtype == torch.bfloat16 else fa2.F32
    outs = []
    for noalloc in (False, True):
        o = torch.full(q.shape, float("nan"), dtype=o_dtype, device=DEV)
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        common = (q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv, n_q, d,
                  scale, table.data_ptr(), table.shape[1], ctx.data_ptr(), max_ctx, page, n_pages, split)
        if noalloc:
            st = fa2.fa2_decode_paged_noalloc(*common, stream.cuda_stream, fa2.BF16, code)
        else:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
            st = fa2.fa2_decode_paged(*common, ws.data_ptr(), ws_bytes, stream.cuda_stream, fa2.BF16, code)
        assert st == fa2.FA2_OK, fa2.fa2_strerror(st)
        outs.append((o, lse))
    stream.synchronize()
    return outs


def _check(outs, what):
    (o1, l1), (o2, l2) = outs
    assert not torch.isnan(o1).any().item() and not torch.isnan(l1).any().item(), what
    same_o = torch.equal(o1.view(torch.int16 if o1.dtype == torch.bfloat16 else torch.int32),
                         o2.view(torch.int16 if o2.dtype == torch.bfloat16 else torch.int32))
    same_l = torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    print(f"[no-alloc] {what}: o bitwise {same_o}, lse bitwise {same_l}", flush=True)
    assert same_o and same_l, what


@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry_point_twice(o_dtype):
    stream = torch.cuda.Stream(device=DEV)
    g = torch.Generator().manual_seed(0)
    lens = torch.randint(1024, 8193, (64,), generator=g).tolist()
    print(f"[case] no-alloc decode, serving batch of 64 sequences, {sum(lens)} keys, o {o_dtype}", flush=True)
    big = _batch(lens, 32, 8, 1, 128, 64, seed=5)
    _check(_both(*big, max(lens), o_dtype, stream), "serving batch")
    print("[case] no-alloc decode, second call: 3 ragged sequences, 4 new tokens, d = 64", flush=True)
    small_lens = [0, 3, 700]
    small = _batch(small_lens, 8, 2, 4, 64, 128, seed=6)
    _check(_both(*small, max(small_lens), o_dtype, stream), "smaller batch after the serving batch")


def test_noalloc_refuses_more_than_the_scratch():
    print("[case] no-alloc decode beyond the scratch", flush=True)
    lens = [1024] * 64
    q, kc, vc, table, ctx = _batch(lens, 32, 8, 1, 128, 64, seed=7)
    o = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    need = fa2.fa2_decode_paged_workspace(64, 32, 8, 1, 128, 1024, 64, 0)[1]
    assert need > fa2.FA2_DECODE_SCRATCH_BYTES
    st = fa2.fa2_decode_paged_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      64, 32, 8, 1, 128, 0.088, table.data_ptr(), table.shape[1], ctx.data_ptr(),
                                      1024, 64, kc.shape[0], 64, 0, fa2.BF16, fa2.F32)
    assert st == fa2.FA2_ERR_SCRATCH
    torch.cuda.synchronize()
