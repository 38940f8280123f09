"""Host-side logic of bench.py (no GPU): the one-GPU exit, the repetition summary and its
spread guard, the algorithmic byte and flop counts against the per-unit figures of the
measurement table (decode 276,897,792 B per step: S 268,435,456 + qkv 1,048,576 + conv
state read and written 6,291,456 + conv weight 65,536 + gate and beta 8,192 + o 1,048,576;
prefill L = 4096 139,100,160 B per call; 8·C·d + 6·d² MFMA flops per (token, V head) with
the Gram products shared by a GQA pair), the counter scaling, and that the committed HBM
counters were taken from the current kernel sources."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import gdn_inputs as gi  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_summary_median_spread_and_guard():
    s = bench.summary([1.00, 1.02, 1.01, 1.03, 1.00])
    assert s["reps"] == 5 and s["median_us"] == pytest.approx(1010.0)
    assert s["spread"] == pytest.approx(0.03 / 1.01) and s["trustworthy"]
    s = bench.summary([1.00, 1.05, 1.01])
    assert s["spread"] == pytest.approx(0.05 / 1.01) and not s["trustworthy"]


def test_algorithmic_bytes_match_the_published_breakdown():
    sh = gi.QWEN
    assert bench.decode_bytes(sh, 64, False) == 268435456 + 1048576 + 6291456 + 65536 + 8192 + 1048576
    assert bench.decode_bytes(sh, 64, False) == 276897792
    assert bench.prefill_bytes(sh, 4096, 1, False) == 139100160


def test_prefill_flops_per_token_head():
    C, d = 64, 128
    assert bench.PREFILL_FLOP_PER_TOKEN_HEAD == 8 * C * d + 6 * d * d == 163840


def test_traffic_scaling_by_the_calibration_copy():
    c = {"fetch_kib_per_dispatch": 1000.0, "write_kib_per_dispatch": 300.0,
         "copy_read_bytes": 268435456, "copy_fetch_kib": 131072.0,       # FETCH_SIZE reads half the copy
         "copy_write_bytes": 268435456, "copy_write_kib": 262144.0}      # WRITE_SIZE all of it
    assert bench.traffic_from_counters(c) == pytest.approx(1000 * 1024 * 2 + 300 * 1024)
    assert bench.traffic_from_counters(None) is None


@pytest.mark.parametrize("name,files", [
    ("decode_B64_d128", ["gdn_recurrent.hip", "gdn_common.hpp"]),
    ("decode_fused_B64_d128", ["gdn_recurrent.hip", "gdn_common.hpp"]),
    ("verify_B128_T4_d128", ["gdn_recurrent.hip", "gdn_common.hpp"]),
    ("prefill_L4096_d128", bench.PREFILL_SOURCES),
    ("ragged_prefill_8seqs_d128", bench.PREFILL_SOURCES),
])
def test_committed_counters_match_the_current_sources(name, files):
    """bench.py reports counter-derived traffic only for counters taken from the sources it
    runs; the committed ones must be current."""
    c = bench.counters(name, bench.source_digest(files))
    assert c is not None, f"profiles/{name}_counters.json was taken from other kernel sources"
    assert c["fetch_kib_per_dispatch"] > 0 and c["write_kib_per_dispatch"] > 0
