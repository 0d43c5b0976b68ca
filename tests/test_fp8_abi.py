"""FP8 entry points on the CPU: argument checks before any HIP call."""

import pytest

import exact_tiled_attention_33_amd as fa2

X, C, S, W, O, L, V, QS, KS = (0x10000000 * (i + 1) for i in range(9))


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def _pack(**over):
    a = dict(x=X, B=2, H=3, N=500, d=128, signs=[1.0] * 128, codes=C, scales=S, ws=W, ws_bytes=1 << 16, stream=0)
    a.update(over)
    return fa2.fa2_fp8_pack(a["x"], a["B"], a["H"], a["N"], a["d"], a["signs"], a["codes"], a["scales"], a["ws"],
                            a["ws_bytes"], a["stream"])


def test_pack_workspace():
    assert fa2.fa2_fp8_pack_workspace(2, 3, 500) == 2 * 3 * 2 * 4
    with pytest.raises(fa2.Fa2Error):
        fa2.fa2_fp8_pack_workspace(0, 3, 500)


@pytest.mark.parametrize("over, status", [
    (dict(x=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws_bytes=2 * 3 * 2 * 4 - 1), fa2.FA2_ERR_INVALID_ARG),
    (dict(d=96, signs=[1.0] * 96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(signs=[1.0] * 127 + [0.5]), fa2.FA2_ERR_INVALID_ARG),
    (dict(codes=X + 1000), fa2.FA2_ERR_INVALID_ARG),   # overlaps x
    (dict(codes=C + 8), fa2.FA2_ERR_INVALID_ARG),      # misaligned
    (dict(N=0), fa2.FA2_ERR_INVALID_ARG),
])
def test_pack_validation(over, status):
    assert _pack(**over) == status


def _fwd(**over):
    a = dict(q8=X, qs=QS, k8=C, ks=KS, v=V, o=O, lse=L, B=1, H=4, Hkv=2, N=1024, d=128, causal=1, scale=0.1,
             stream=0, o_dtype=fa2.F32)
    a.update(over)
    return fa2.fa2_fwd_fp8(a["q8"], a["qs"], a["k8"], a["ks"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                           a["N"], a["d"], a["causal"], a["scale"], a["stream"], a["o_dtype"])


@pytest.mark.parametrize("over, status", [
    (dict(q8=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(qs=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(causal=2), fa2.FA2_ERR_INVALID_ARG),
    (dict(Hkv=3), fa2.FA2_ERR_INVALID_ARG),
    (dict(d=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), fa2.FA2_ERR_INVALID_ARG),
    (dict(o=X + 64), fa2.FA2_ERR_INVALID_ARG),      # o overlaps q8
    (dict(lse=V + 4), fa2.FA2_ERR_INVALID_ARG),     # lse overlaps v
    (dict(o_dtype=5), fa2.FA2_ERR_INVALID_ARG),
])
def test_fwd_fp8_validation(over, status):
    assert _fwd(**over) == status


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_no_device_status_on_cpu_only_host():
    assert _pack() == fa2.FA2_ERR_NO_DEVICE
    assert _pack(signs=None) == fa2.FA2_ERR_NO_DEVICE
    assert _fwd() == fa2.FA2_ERR_NO_DEVICE
    assert _fwd(causal=0, d=64, o_dtype=fa2.BF16) == fa2.FA2_ERR_NO_DEVICE
