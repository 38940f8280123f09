"""The seeded input generators draw the same tensors as when the stored digests were
written (tests/golden/make_input_hashes.py): the workloads are reproducible seed by seed,
and the ragged workload's sequence lengths are the ones the design notes quote."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_input_hashes as mih  # noqa: E402

import gdn_inputs as gi  # noqa: E402


def test_generator_digests():
    with open(os.path.join(HERE, "golden", "input_hashes.json")) as f:
        stored = json.load(f)
    got = {k: mih.digest(v) for k, v in mih.cases().items()}
    assert got.keys() == stored.keys()
    bad = [k for k in got if got[k] != stored[k]]
    assert not bad, bad


def test_ragged_lengths_and_reproducibility():
    lens = gi.seq_lens(gi.RAGGED_N, gi.RAGGED_LO, gi.RAGGED_HI, gi.WORKLOADS[3].seed)
    assert int(lens.sum()) == 28457 and lens.min() >= 512 and lens.max() <= 8192
    a = gi.qkv(gi.QWEN, 1, 8, 1234, "bf16")
    assert np.array_equal(a, gi.qkv(gi.QWEN, 1, 8, 1234, "bf16"))
    assert not np.array_equal(a, gi.qkv(gi.QWEN, 1, 8, 1235, "bf16"))
