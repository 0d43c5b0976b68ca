"""fa2_decode_paged and its workspace helper on the CPU: chunk choice,
workspace arithmetic, and rejection of malformed calls before any HIP
call.  No compute call is made here."""

import pytest

import exact_tiled_attention_33_amd as fa2


def test_workspace_helper():
    # groups of 4 rows (one wavefront per chunk): 256 groups on 256 units:
    # 1024 wavefront slots, four chunks of 2048 keys for an 8192-key context
    assert fa2.fa2_decode_paged_workspace(32, 32, 8, 1, 128, 8192, 0, 256) == (2048, 32 * 8 * 4 * 4 * 1 * (128 * 4 + 8))
    # 512 groups: two chunks of 4096 keys; 16 x 8 = 128 groups: eight of 1024
    assert fa2.fa2_decode_paged_workspace(64, 32, 8, 1, 128, 8192, 0, 256)[0] == 4096
    assert fa2.fa2_decode_paged_workspace(16, 32, 8, 1, 128, 8192, 0, 256)[0] == 1024
    # the groups alone fill the slots: four chunks per sequence
    assert fa2.fa2_decode_paged_workspace(256, 32, 8, 1, 128, 8192, 0, 256)[0] == 2048
    # groups of 64 rows: two wavefronts (row blocks) per chunk and group; at
    # least 256 keys per chunk
    assert fa2.fa2_decode_paged_workspace(4, 64, 1, 1, 128, 8192, 0, 256)[0] == 256
    assert fa2.fa2_decode_paged_workspace(1, 64, 1, 1, 128, 1 << 20, 0, 256)[0] == 2048
    # groups of 256 rows (forward kernel workgroups): about eight per unit
    assert fa2.fa2_decode_paged_workspace(1, 256, 1, 1, 128, 1 << 20, 0, 256)[0] == 512
    # a short context: one chunk covering it
    sk, ws = fa2.fa2_decode_paged_workspace(1, 8, 1, 1, 128, 100, 0, 256)
    assert sk == 128 and ws == 1 * 1 * 1 * 8 * (128 * 4 + 8)
    # an explicit chunk is kept
    sk, ws = fa2.fa2_decode_paged_workspace(2, 4, 2, 3, 64, 1000, 192, 0)
    assert sk == 192 and ws == 2 * 2 * 6 * 2 * 3 * (64 * 4 + 8)


@pytest.mark.parametrize("args, status", [
    ((1, 4, 3, 1, 128, 100, 0, 256), fa2.FA2_ERR_INVALID_ARG),    # H_kv does not divide H
    ((1, 4, 2, 0, 128, 100, 0, 256), fa2.FA2_ERR_INVALID_ARG),    # no new token
    ((1, 4, 2, 1, 128, 0, 0, 256), fa2.FA2_ERR_INVALID_ARG),      # no context bound
    ((1, 4, 2, 1, 128, 100, 100, 256), fa2.FA2_ERR_INVALID_ARG),  # chunk not a multiple of 64
    ((1, 4, 2, 1, 128, 100, 0, 0), fa2.FA2_ERR_INVALID_ARG),      # library's choice needs the unit count
    ((1, 4, 2, 1, 96, 100, 0, 256), fa2.FA2_ERR_UNSUPPORTED),
    ((1, 64, 1, 5, 128, 100, 0, 256), fa2.FA2_ERR_UNSUPPORTED),   # 320 query rows per key/value head
])
def test_workspace_helper_rejections(args, status):
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.fa2_decode_paged_workspace(*args)
    assert e.value.status == status


Q, KC, VC, O, L, PT, CL, W = (0x10000000 * (i + 1) for i in range(8))
GOOD = dict(q=Q, kc=KC, vc=VC, o=O, lse=L, B=2, H=8, Hkv=2, n_q=1, d=128, scale=0.1, pt=PT, max_pages=4, cl=CL,
            max_ctx=256, page=64, n_pages=8, split=128, ws=W, ws_bytes=1 << 20, stream=0, in_dtype=fa2.BF16,
            o_dtype=fa2.F32)


def _call(**over):
    a = dict(GOOD, **over)
    return fa2.fa2_decode_paged(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["n_q"],
                                a["d"], a["scale"], a["pt"], a["max_pages"], a["cl"], a["max_ctx"], a["page"],
                                a["n_pages"], a["split"], a["ws"], a["ws_bytes"], a["stream"], a["in_dtype"],
                                a["o_dtype"])


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.parametrize("over, status", [
    (dict(q=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(pt=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(cl=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws_bytes=2 * 2 * 2 * 4 * (128 * 4 + 8) - 1), fa2.FA2_ERR_INVALID_ARG),
    (dict(split=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(split=100), fa2.FA2_ERR_INVALID_ARG),
    (dict(page=32), fa2.FA2_ERR_UNSUPPORTED),
    (dict(page=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(max_pages=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(n_pages=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(in_dtype=fa2.F32), fa2.FA2_ERR_UNSUPPORTED),
    (dict(o_dtype=7), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa2.FA2_ERR_INVALID_ARG),
    (dict(Hkv=3), fa2.FA2_ERR_INVALID_ARG),
    (dict(n_q=129), fa2.FA2_ERR_UNSUPPORTED),
    (dict(pt=PT + 2), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws=W + 4), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws=O), fa2.FA2_ERR_INVALID_ARG),          # workspace overlaps o
    (dict(o=KC + 64), fa2.FA2_ERR_INVALID_ARG),      # o inside the key cache
    (dict(lse=CL), fa2.FA2_ERR_INVALID_ARG),         # lse overlaps the context lengths
])
def test_decode_validation(over, status):
    assert _call(**over) == status


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_decode_no_device_status_on_cpu_only_host():
    assert _call() == fa2.FA2_ERR_NO_DEVICE
    assert _call(n_q=4, split=64, page=256, o_dtype=fa2.BF16) == fa2.FA2_ERR_NO_DEVICE


# --- fa2_decode_paged_noalloc: the same checks, no workspace argument -------

def _call_noalloc(**over):
    a = dict(GOOD, **over)
    return fa2.fa2_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                                        a["n_q"], a["d"], a["scale"], a["pt"], a["max_pages"], a["cl"],
                                        a["max_ctx"], a["page"], a["n_pages"], a["split"], a["stream"],
                                        a["in_dtype"], a["o_dtype"])


@pytest.mark.parametrize("over, status", [
    (dict(q=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(pt=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(split=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(split=100), fa2.FA2_ERR_INVALID_ARG),
    (dict(page=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(in_dtype=fa2.F32), fa2.FA2_ERR_UNSUPPORTED),
    (dict(o=KC + 64), fa2.FA2_ERR_INVALID_ARG),
    (dict(lse=CL), fa2.FA2_ERR_INVALID_ARG),
    (dict(pt=PT + 2), fa2.FA2_ERR_INVALID_ARG),
])
def test_noalloc_validation(over, status):
    assert _call_noalloc(**over) == status


# 64 sequences x 32 query heads, one new token, d = 128: 2048 rows of
# 128*4 + 8 bytes per 64-key chunk; 16 chunks need 17,039,360 bytes.
BIG = dict(B=64, H=32, Hkv=8, n_q=1, d=128, split=64, max_pages=16, page=64, n_pages=1024)


def test_noalloc_rejects_more_than_the_scratch():
    need = fa2.fa2_decode_paged_workspace(64, 32, 8, 1, 128, 1024, 64, 0)[1]
    assert need == 16 * 2048 * (128 * 4 + 8) > fa2.FA2_DECODE_SCRATCH_BYTES
    assert _call_noalloc(max_ctx=1024, **BIG) == fa2.FA2_ERR_SCRATCH
    assert "scratch" in fa2.fa2_strerror(fa2.FA2_ERR_SCRATCH)


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_noalloc_no_device_status_on_cpu_only_host():
    assert _call_noalloc() == fa2.FA2_ERR_NO_DEVICE
    # 15 chunks (15,974,400 bytes) fit in the scratch
    assert fa2.fa2_decode_paged_workspace(64, 32, 8, 1, 128, 960, 64, 0)[1] <= fa2.FA2_DECODE_SCRATCH_BYTES
    assert _call_noalloc(max_ctx=960, **BIG) == fa2.FA2_ERR_NO_DEVICE
