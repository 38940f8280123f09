"""The host-side bounds model of the prefill carry (tests/carry_model.cpp), built with g++
against the index header the kernels compute their addresses from. It replays every
carry workgroup of every launch configuration the launcher can choose (segment 0's weight
4..7 eighths, 32..256 CUs, unpacked and packed prompts) and checks every global offset
and LDS slot, the barrier counts of the loader and compute waves, and the state-map
prologue's vmcnt waits. Four planted mistakes must each be reported."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("carry_model") / "carry_model")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror",
                           "-I", os.path.join(ROOT, "linear_attention_sequence_amd", "csrc"),
                           os.path.join(HERE, "carry_model.cpp"), "-o", exe])
    return exe


def test_every_carry_launch_stays_in_bounds(model):
    r = subprocess.run([model], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "all hold" in r.stdout, r.stdout


@pytest.mark.parametrize("plant", ["wait32", "loader_barrier", "tail_row", "seg0_wide"])
def test_planted_mistakes_are_reported(model, plant):
    r = subprocess.run([model, plant], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1 and "VIOLATION" in r.stderr, (plant, r.stdout, r.stderr)
