"""The C-ABI library on the CPU: it loads, exports what include/fa2.h
declares, rejects malformed calls before any HIP call, and its grid
arithmetic reproduces the counts the pages print.

No compute call is made here.  The one test that passes valid arguments
(expecting FA2_ERR_NO_DEVICE) is skipped where a GPU is present.
"""

import re
import subprocess
from pathlib import Path

import pytest

import exact_tiled_attention_33_amd as fa2

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "fa2.h"


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(fa2.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = fa2.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(fa2.library_path())],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name


def test_version_matches_header():
    m = re.search(r"#define FA2_VERSION (\d+)", HEADER.read_text())
    assert fa2.fa2_version() == int(m.group(1))


def test_status_codes_match_header():
    text = HEADER.read_text()
    for name in ("FA2_OK", "FA2_ERR_INVALID_ARG", "FA2_ERR_UNSUPPORTED", "FA2_ERR_NO_DEVICE", "FA2_ERR_LAUNCH",
                 "FA2_ERR_SCRATCH"):
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
        assert int(m.group(1)) == getattr(fa2, name), name
    m = re.search(r"#define FA2_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert int(m.group(1)) << int(m.group(2)) == fa2.FA2_DECODE_SCRATCH_BYTES
    for name in ("F32", "BF16"):
        m = re.search(rf"\bFA2_{name}\s*=\s*(\d+)", text)
        assert int(m.group(1)) == getattr(fa2, name)


def test_strerror():
    for st in (fa2.FA2_OK, fa2.FA2_ERR_INVALID_ARG, fa2.FA2_ERR_UNSUPPORTED, fa2.FA2_ERR_NO_DEVICE,
               fa2.FA2_ERR_LAUNCH, fa2.FA2_ERR_SCRATCH, 12345):
        assert isinstance(fa2.fa2_strerror(st), str) and fa2.fa2_strerror(st)
    assert fa2.fa2_strerror(12345) == "unknown status"


# Fake, distinct, 256-byte aligned "device" addresses: never dereferenced,
# because every call below fails validation first.
Q, K, V, O, L = (0x10000000 * (i + 1) for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=64, d=64, causal=0, scale=0.125,
            stream=0, in_dtype=fa2.BF16, o_dtype=fa2.F32)


def _call(**over):
    a = dict(GOOD, **over)
    return fa2.fa2_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                       a["causal"], a["scale"], a["stream"], a["in_dtype"], a["o_dtype"])


@pytest.mark.parametrize("over, status", [
    (dict(q=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(k=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(v=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(o=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(lse=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(B=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(H=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(N=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(d=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(d=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(d=256), fa2.FA2_ERR_UNSUPPORTED),
    (dict(causal=2), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa2.FA2_ERR_INVALID_ARG),
    (dict(in_dtype=7), fa2.FA2_ERR_INVALID_ARG),
    (dict(o_dtype=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(q=Q + 8), fa2.FA2_ERR_INVALID_ARG),
    (dict(o=O + 4), fa2.FA2_ERR_INVALID_ARG),
    (dict(lse=L + 2), fa2.FA2_ERR_INVALID_ARG),
    (dict(o=Q + 64), fa2.FA2_ERR_INVALID_ARG),      # output overlaps q
    (dict(lse=V + 16), fa2.FA2_ERR_INVALID_ARG),    # lse overlaps v
    (dict(lse=O + 16), fa2.FA2_ERR_INVALID_ARG),    # lse overlaps o
    (dict(B=1 << 20, H=1 << 20, N=1 << 20), fa2.FA2_ERR_INVALID_ARG),  # > 2^60 elements
])
def test_validation_rejects_before_any_hip_call(over, status):
    assert _call(**over) == status


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_no_device_status_on_cpu_only_host():
    assert _call() == fa2.FA2_ERR_NO_DEVICE


def test_forward_without_gpu_raises():
    import torch
    if _gpu_present():
        pytest.skip("GPU present")
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa2.forward(q, q, q)


# --- grid arithmetic: the pages' counts (Saraf, section 2.2 and 2.3) -------

def test_pages_block_counts_a100():
    # two 8192-token sequences x 16 heads, 64-row query blocks, 108 SMs
    per_head = fa2.fa2_plan(2, 16, 8192, 128, 0, fa2.BF16, block_rows=8192, block_cols=64, num_units=108)
    assert per_head["workgroups"] == 32                       # one block per (sequence, head)
    assert per_head["last_wave_groups"] == 32                  # 76 of 108 SMs idle
    seq = fa2.fa2_plan(2, 16, 8192, 128, 0, fa2.BF16, block_rows=64, block_cols=64, num_units=108)
    assert seq["query_tiles"] == 128
    assert seq["workgroups"] == 4096
    assert round(seq["waves_of_groups"], 1) == 37.9
    assert seq["last_wave_groups"] == 100                     # 8 of 108 idle in the last wave
    # one division per query block: 128 per head, against one per (query, key) block pair
    assert seq["normalisations"] // 32 == 128
    assert seq["tile_pairs"] // 32 == 16384


def test_pages_score_matrix_size():
    # a 16-bit score matrix for one head at 8192 tokens is 128 MiB
    assert 8192 * 8192 * 2 == 128 * 2**20


def test_own_plan_for_the_workloads():
    import workloads
    mi355x_cus = 256
    # bf16 and fp32 alike: 128-row query tiles
    expect_groups = {"fp32_small": 1, "short_seq": 2048, "mid_seq": 2048, "long_causal": 2048,
                     "long_few_head": 512}
    for name, w in workloads.WORKLOADS.items():
        code = fa2.BF16 if w.dtype == "bf16" else fa2.F32
        p = fa2.fa2_plan(w.B, w.H, w.N, w.d, int(w.causal), code, num_units=mi355x_cus)
        assert p["workgroups"] == expect_groups[name], name
        assert p["flops_credited"] == workloads.credited_flops(w.B, w.H, w.N, w.d, w.causal)
        assert p["flops_executed"] >= p["flops_credited"]
        if w.causal:
            # above-diagonal key tiles are skipped: executed work stays within 4% of credited
            assert p["flops_executed"] / p["flops_credited"] < 1.04, name
        else:
            assert p["flops_executed"] == p["flops_credited"]


def test_plan_rejects_what_fwd_rejects():
    with pytest.raises(fa2.Fa2Error):
        fa2.fa2_plan(1, 1, 0, 64, 0, fa2.BF16)
    with pytest.raises(fa2.Fa2Error):
        fa2.fa2_plan(1, 1, 8, 80, 0, fa2.BF16)
    with pytest.raises(fa2.Fa2Error):
        fa2.fa2_plan(1, 1, 8, 64, 3, fa2.BF16)


# --- fa2_bwd argument validation (no compute) --------------------------------

BQ, BK, BV, BO, BG, BL, BD, DQ, DK, DV = (0x10000000 * (i + 1) for i in range(10))
BGOOD = dict(q=BQ, k=BK, v=BV, o=BO, dout=BG, lse=BL, delta=BD, dq=DQ, dk=DK, dv=DV, B=1, H=2,
             N=64, d=128, causal=1, scale=0.088, stream=0, in_dtype=fa2.BF16, o_dtype=fa2.F32,
             grad_dtype=fa2.F32)


def _bcall(**over):
    a = dict(BGOOD, **over)
    return fa2.fa2_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["delta"], a["dq"],
                       a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"],
                       a["stream"], a["in_dtype"], a["o_dtype"], a["grad_dtype"])


@pytest.mark.parametrize("over, status", [
    *[(dict(**{name: 0}), fa2.FA2_ERR_INVALID_ARG)
      for name in ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk", "dv")],
    (dict(B=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(N=-3), fa2.FA2_ERR_INVALID_ARG),
    (dict(causal=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa2.FA2_ERR_INVALID_ARG),
    (dict(o_dtype=9), fa2.FA2_ERR_INVALID_ARG),
    (dict(grad_dtype=2), fa2.FA2_ERR_INVALID_ARG),
    (dict(in_dtype=5), fa2.FA2_ERR_INVALID_ARG),
    (dict(dq=DQ + 8), fa2.FA2_ERR_INVALID_ARG),     # misaligned output
    (dict(delta=BD + 2), fa2.FA2_ERR_INVALID_ARG),  # misaligned workspace
    (dict(dk=BQ + 256), fa2.FA2_ERR_INVALID_ARG),   # output overlaps q
    (dict(dv=DK + 64), fa2.FA2_ERR_INVALID_ARG),    # outputs overlap each other
    (dict(delta=BL + 4), fa2.FA2_ERR_INVALID_ARG),  # workspace overlaps lse
    (dict(delta=DV + 16), fa2.FA2_ERR_INVALID_ARG),  # workspace overlaps an output
    (dict(d=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(d=256), fa2.FA2_ERR_UNSUPPORTED),
    (dict(in_dtype=fa2.F32), fa2.FA2_ERR_UNSUPPORTED),
])
def test_bwd_validation_rejects_before_any_hip_call(over, status):
    assert _bcall(**over) == status


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_bwd_no_device_status_on_cpu_only_host():
    assert _bcall() == fa2.FA2_ERR_NO_DEVICE
    assert _bcall(grad_dtype=fa2.BF16, o_dtype=fa2.BF16, causal=0) == fa2.FA2_ERR_NO_DEVICE


# --- grouped key/value heads (fa2_fwd_gqa, fa2_bwd_gqa) ----------------------

def _gcall(H=8, H_kv=2, **over):
    a = dict(GOOD, H=H, **over)
    return fa2.fa2_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], H_kv, a["N"],
                           a["d"], a["causal"], a["scale"], a["stream"], a["in_dtype"], a["o_dtype"])


def _gbcall(H=8, H_kv=2, **over):
    a = dict(BGOOD, H=H, **over)
    return fa2.fa2_bwd_gqa(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["delta"], a["dq"],
                           a["dk"], a["dv"], a["B"], a["H"], H_kv, a["N"], a["d"], a["causal"],
                           a["scale"], a["stream"], a["in_dtype"], a["o_dtype"], a["grad_dtype"])


@pytest.mark.parametrize("H, H_kv", [(8, 0), (8, -2), (8, 3), (6, 4), (4, 8)])
def test_gqa_rejects_head_counts_that_do_not_divide(H, H_kv):
    assert _gcall(H=H, H_kv=H_kv) == fa2.FA2_ERR_INVALID_ARG
    assert _gbcall(H=H, H_kv=H_kv) == fa2.FA2_ERR_INVALID_ARG


def test_gqa_overlap_checks_use_the_key_value_sizes():
    # q, o: 1 x 8 x 64 x 64 bf16/fp32; k, v: 1 x 2 x 64 x 64 bf16 = 16 KiB each
    kv_bytes = 1 * 2 * 64 * 64 * 2
    assert _gcall(o=K + kv_bytes - 16) == fa2.FA2_ERR_INVALID_ARG   # o starts inside k
    bkv = 1 * 2 * 64 * 128 * 4                                       # dk fp32
    assert _gbcall(dv=DK + bkv - 16) == fa2.FA2_ERR_INVALID_ARG      # dv starts inside dk


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_gqa_no_device_status_on_cpu_only_host():
    assert _gcall() == fa2.FA2_ERR_NO_DEVICE
    assert _gcall(H=8, H_kv=1) == fa2.FA2_ERR_NO_DEVICE
    assert _gbcall() == fa2.FA2_ERR_NO_DEVICE
    # o right after the (smaller) key buffer does not overlap it
    assert _gcall(o=K + 1 * 2 * 64 * 64 * 2) == fa2.FA2_ERR_NO_DEVICE


# --- sliding-window forward (fa2_fwd_window) ---------------------------------

def _wcall(wl, wr, **over):
    a = dict(GOOD, **over)
    return fa2.fa2_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H"], a["N"],
                              a["d"], wl, wr, a["scale"], a["stream"], a["in_dtype"], a["o_dtype"])


@pytest.mark.parametrize("wl, wr", [(-2, 0), (0, -3), (-5, -5)])
def test_window_rejects_bounds_below_minus_one(wl, wr):
    assert _wcall(wl, wr) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("wl, wr", [(0, 0), (10, 0), (-1, 5), (3, 3)])
def test_window_fp32_supports_only_no_mask_and_causal(wl, wr):
    assert _wcall(wl, wr, in_dtype=fa2.F32) == fa2.FA2_ERR_UNSUPPORTED


@pytest.mark.skipif(_gpu_present(), reason="valid fake pointers would launch on a real GPU")
def test_window_no_device_status_on_cpu_only_host():
    for wl, wr in ((-1, -1), (-1, 0), (0, 0), (100, 7)):
        assert _wcall(wl, wr) == fa2.FA2_ERR_NO_DEVICE
    # bounds of N or more are no bounds: fp32 accepts them as no mask / causal
    assert _wcall(64, 0, in_dtype=fa2.F32) == fa2.FA2_ERR_NO_DEVICE
    assert _wcall(1000, 1000, in_dtype=fa2.F32) == fa2.FA2_ERR_NO_DEVICE


def _wbcall(wl, wr, **over):
    a = dict(BGOOD, **over)
    return fa2.fa2_bwd_window(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["delta"], a["dq"],
                              a["dk"], a["dv"], a["B"], a["H"], a["H"], a["N"], a["d"], wl, wr, a["scale"],
                              a["stream"], a["in_dtype"], a["o_dtype"], a["grad_dtype"])


def test_bwd_window_validation():
    assert _wbcall(-2, 0) == fa2.FA2_ERR_INVALID_ARG
    assert _wbcall(0, -7) == fa2.FA2_ERR_INVALID_ARG
    assert _wbcall(5, 5, d=96) == fa2.FA2_ERR_UNSUPPORTED
    if not _gpu_present():
        assert _wbcall(5, 5) == fa2.FA2_ERR_NO_DEVICE
        assert _wbcall(5, 5, d=64) == fa2.FA2_ERR_NO_DEVICE
        assert _wbcall(-1, 0) == fa2.FA2_ERR_NO_DEVICE


# --- the shader-clock probe (a benchmark diagnostic) -------------------------

@pytest.mark.parametrize("groups, ticks, out", [(0, 10, 0x10000000), (65537, 10, 0x10000000), (4, 0, 0x10000000),
                                                (4, 10**9 + 1, 0x10000000), (4, 10, 0), (4, 10, 0x10000004)])
def test_clock_probe_rejects_before_any_hip_call(groups, ticks, out):
    assert fa2.fa2_clock_probe(groups, ticks, out, 0) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.skipif(_gpu_present(), reason="a valid fake pointer would launch on a real GPU")
def test_clock_probe_no_device_status_on_cpu_only_host():
    assert fa2.fa2_clock_probe(4, 10, 0x10000000, 0) == fa2.FA2_ERR_NO_DEVICE
