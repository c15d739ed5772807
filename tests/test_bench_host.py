"""Host-side parts of bench.py (no GPU): the exit for more than one GPU, the
source hash that guards committed counter summaries, and the CPU-oracle
baselines of the table workloads on small shapes."""

import dataclasses
import json
import subprocess
import sys
import os

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_source_hash_is_stable_and_covers_the_kernels():
    h1, h2 = bench.source_hash(), bench.source_hash()
    assert h1 == h2 and len(h1) >= 16
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, f)), f


def test_committed_counter_summaries_are_well_formed():
    for name in ("fa_fwd_causal_bf16_b4h16n8192d64", "fa_decode_bf16_b64h32d128",
                 "fa_bwd_causal_bf16_b4h16n8192d64"):
        d = json.load(open(os.path.join(ROOT, "profiles", name + ".counters.json")))
        assert d["hbm_bytes_per_launch"] > 0
        assert "source_hash" in d


def _check(cb, unit):
    assert cb["kind"] == "oracle" and cb["unit"] == unit
    assert cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]


def test_cpu_baseline_prefill():
    _check(bench.cpu_baseline_config(wl.SMALL[2], 0.2), "TFLOP/s")


def test_cpu_baseline_varlen_and_decode():
    _check(bench.cpu_baseline_config(wl.SMALL[4], 0.2), "TFLOP/s")
    _check(bench.cpu_baseline_config(dataclasses.replace(wl.SMALL[5], B=2), 0.2), "GB/s")


def test_cpu_baseline_skips_workloads_it_does_not_cover():
    assert bench.cpu_baseline_config(dataclasses.replace(wl.SMALL[3], backward=True), 0.1) is None
