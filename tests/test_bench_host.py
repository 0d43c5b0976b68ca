"""bench.py on the host (no GPU): the HBM-traffic lookup from profiles/
(a counter summary counts only while its source stamp matches), the
committed summaries against the committed kernel sources, and the refusal
of more than one GPU."""

import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_profile(tmp_path, name, stamp, nbytes):
    (tmp_path / "profiles").mkdir(exist_ok=True)
    (tmp_path / "profiles" / f"{name}_hbm.md").write_text(
        f"# summary\n\nkernel_source_sha256_16: {stamp}\n\nhbm_bytes_per_launch: {nbytes}\n")


def test_traffic_counts_only_with_a_matching_stamp(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "0123456789abcdef")
    _write_profile(tmp_path, "fa2_fwd_toy", "0123456789abcdef", "42.5e6")
    assert bench.traffic_from_profiles("toy") == 42.5e6
    _write_profile(tmp_path, "fa2_fwd_toy", "fedcba9876543210", "42.5e6")
    assert bench.traffic_from_profiles("toy") is None
    assert bench.traffic_from_profiles("missing") is None


def test_traffic_profile_name_and_sources(tmp_path, monkeypatch):
    seen = []

    def fake_hash(sources=None):
        seen.append(sources)
        return "aaaaaaaaaaaaaaaa"

    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", fake_hash)
    _write_profile(tmp_path, "fa2_decode_paged", "aaaaaaaaaaaaaaaa", "1382.4e6")
    assert bench.traffic_from_profiles("paged_decode", "fa2_decode_paged", bench.DECODE_SOURCES) == 1382.4e6
    assert seen[-1] == bench.DECODE_SOURCES


@pytest.mark.parametrize("args", [
    ("long_causal", None, None),
    ("short_seq", None, None),
    ("paged_decode", "fa2_decode_paged", "DECODE_SOURCES"),
    ("long_causal", "fa2_bwd_long_causal", "BWD_SOURCES"),
])
def test_committed_counter_summaries_match_the_sources(args):
    # the counter summaries under profiles/ were measured on the kernel
    # sources as committed: a kernel change must come with new counters
    workload, profile, sources = args
    src = getattr(bench, sources) if sources else None
    assert bench.traffic_from_profiles(workload, profile, src) is not None, (
        f"profiles/{profile or 'fa2_fwd_' + workload}_hbm.md is stamped for other kernel sources")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
