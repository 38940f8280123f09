"""Writes input_hashes.json: SHA-256 digests of tensors drawn by gdn_inputs for fixed
seeds and shapes, so that a change to any generator (distribution, stream id, rounding)
shows up as a failing test instead of as silently different workloads.

Run from the repository root: python tests/golden/make_input_hashes.py
It calls gdn_inputs only (no part of the layer's arithmetic)."""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import gdn_inputs as gi  # noqa: E402


def digest(a) -> str:
    a = np.ascontiguousarray(a)
    h = hashlib.sha256()
    h.update(str(a.dtype).encode() + str(a.shape).encode())
    h.update(a.tobytes())
    return h.hexdigest()


def cases():
    T, Q = gi.TINY, gi.QWEN
    s0, s1, s2, s3, s4 = (gi.WORKLOADS[i].seed for i in range(5))
    return {
        "tiny.qkv": gi.qkv(T, 1, 64, s0, "f32"),
        "tiny.gate": gi.gate(T, 1, 64, s0, "f32"),
        "tiny.beta": gi.beta(T, 1, 64, s0, "f32"),
        "tiny.conv_weight": gi.conv_weight(T, s0, "f32"),
        "decode.qkv.step0": gi.qkv(Q, 64, 1, s1, "bf16", step=0),
        "decode.qkv.step255": gi.qkv(Q, 64, 1, s1, "bf16", step=255),
        "decode.gate.step7": gi.gate(Q, 64, 1, s1, "bf16", step=7),
        "decode.beta.step7": gi.beta(Q, 64, 1, s1, "bf16", step=7),
        "decode.state0": gi.state0(Q, 2, s1, 0.1),
        "decode.conv_state0": gi.conv_state0(Q, 2, s1, 1.0, "bf16"),
        "prefill.qkv.first64": gi.qkv(Q, 1, 64, s2, "bf16"),
        "prefill.conv_weight": gi.conv_weight(Q, s2, "bf16"),
        "ragged.seq_lens": gi.seq_lens(gi.RAGGED_N, gi.RAGGED_LO, gi.RAGGED_HI, s3),
        "ragged.cu_seqlens": gi.cu_seqlens(gi.seq_lens(gi.RAGGED_N, gi.RAGGED_LO, gi.RAGGED_HI, s3)),
        "verify.accept_len": gi.accept_len(gi.VERIFY_B, gi.VERIFY_T, s4),
        "verify.gate": gi.gate(Q, 4, gi.VERIFY_T, s4, "bf16"),
        "fusion.a_raw": gi.a_raw(Q, 1, 16, s2, "bf16"),
        "fusion.b_raw": gi.b_raw(Q, 1, 16, s2, "bf16"),
        "fusion.a_log": gi.a_log(Q, s2, "bf16"),
        "fusion.dt_bias": gi.dt_bias(Q, s2, "bf16"),
        "fusion.z": gi.z_gate(Q, 1, 4, s2, "bf16"),
        "fusion.norm_weight": gi.norm_weight(Q, s2, "bf16"),
    }


if __name__ == "__main__":
    out = {k: digest(v) for k, v in cases().items()}
    with open(os.path.join(HERE, "input_hashes.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {len(out)} digests")
