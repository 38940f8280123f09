"""GPU parity: every entry point of libgdn.so against the fp64 oracle on the same
seeded inputs, plus bit-exact GPU invariants. Needs an MI355X."""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_sequence_amd as gdn
import oracle
from gpu_cases import TOL, dev, layer_inputs, oparams, params, rel_err, run_prefill

pytestmark = pytest.mark.gpu

SMALL128 = gi.Shape(Hk=2, Hv=4, dk=128, dv=128, K=4)   # d = 128 tiles, GQA factor 2


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    oracle.build_oracle(force=False)


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# conv1d + SiLU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape,dtype,B,L", [(gi.TINY, "f32", 1, 64), (SMALL128, "bf16", 2, 300),
                                             (gi.TINY_GQA, "f32", 3, 1)])
def test_conv1d_silu(shape, dtype, B, L):
    _say(f"conv1d_silu {shape} {dtype} B={B} L={L}")
    inp = layer_inputs(shape, B, L, 7, dtype, conv_std=1.0)
    p = params(shape, dtype)
    y = torch.full((B, shape.D, L), float("nan"), device="cuda")
    cout = torch.zeros_like(dev(inp["conv0"], dtype))
    gdn.gdn_conv1d_silu(p, dev(inp["qkv"], dtype), dev(inp["w"], dtype), dev(inp["conv0"], dtype), cout, y)
    torch.cuda.synchronize()
    y_ref, c_ref = oracle.conv1d_silu(oparams(shape), inp["qkv"], inp["w"], inp["conv0"])
    assert rel_err(y, y_ref) <= TOL[dtype]
    assert np.array_equal(cout.float().cpu().numpy(), c_ref)


def test_conv1d_silu_ragged():
    shape, dtype = SMALL128, "bf16"
    lens = [5, 0, 300, 1, 2]
    cu = gi.cu_seqlens(lens)
    Lt = int(cu[-1]) + 7   # 7 trailing tokens owned by no sequence stay untouched
    inp = layer_inputs(shape, 1, Lt, 8, dtype, N=len(lens), conv_std=1.0)
    p = params(shape, dtype)
    y = torch.full((1, shape.D, Lt), 12345.0, device="cuda")
    cout = torch.zeros_like(dev(inp["conv0"], dtype))
    gdn.gdn_conv1d_silu(p, dev(inp["qkv"], dtype), dev(inp["w"], dtype), dev(inp["conv0"], dtype),
                        cout, y, cu_seqlens=dev(cu))
    torch.cuda.synchronize()
    y_ref, c_ref = oracle.conv1d_silu(oparams(shape), inp["qkv"][:, :, :int(cu[-1])], inp["w"],
                                      inp["conv0"], cu_seqlens=cu)
    assert rel_err(y[:, :, :int(cu[-1])], y_ref) <= TOL[dtype]
    assert torch.all(y[:, :, int(cu[-1]):] == 12345.0)
    assert np.array_equal(cout.float().cpu().numpy(), c_ref)


# ---------------------------------------------------------------------------
# prefill, full comparison at small sizes (several chunks and a ragged tail)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape,dtype,B,L,s0", [
    (gi.TINY, "f32", 1, 64, 0.0),
    (gi.TINY_GQA, "f32", 2, 150, 0.1),
    (SMALL128, "bf16", 1, 200, 0.1),
    (SMALL128, "bf16", 2, 1, 0.1),
    (SMALL128, "f32", 1, 129, 0.1),
])
def test_prefill_small(shape, dtype, B, L, s0):
    _say(f"prefill {shape} {dtype} B={B} L={L}")
    inp = layer_inputs(shape, B, L, 11, dtype, s0_std=s0, conv_std=1.0 if s0 else 0.0)
    got = run_prefill(shape, dtype, inp)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]
    assert np.array_equal(got["conv_out"].float().cpu().numpy(), ref["conv_out"])


def test_prefill_ragged_small():
    shape, dtype = SMALL128, "bf16"
    lens = [70, 0, 130, 1, 64]
    cu = gi.cu_seqlens(lens)
    inp = layer_inputs(shape, 1, int(cu[-1]), 12, dtype, N=len(lens), s0_std=0.1, conv_std=1.0)
    got = run_prefill(shape, dtype, inp, cu=cu)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"], cu_seqlens=cu)
    assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]
    assert np.array_equal(got["conv_out"].float().cpu().numpy(), ref["conv_out"])


@pytest.mark.parametrize("B,L", [(2, 150), (5, 130), (2, 800)], ids=["split_heads_B2", "whole_heads_B5", "segments_B2"])
def test_prefill_carry_launch_paths(B, L):
    """The full 16/32-head, d = 128 shape unpacked: B = 2 (64 heads) runs the carry with two
    workgroups per head and a loader wave, and in 3 segments once it has 12 chunks (800
    tokens); B = 5 (160 heads, more than half the CUs' worth of half-head workgroups) runs
    whole-head workgroups of 8 waves."""
    shape, dtype = gi.QWEN, "bf16"
    _say(f"prefill carry path B={B} L={L}")
    inp = layer_inputs(shape, B, L, 14 + B, dtype, s0_std=0.1, conv_std=1.0)
    got = run_prefill(shape, dtype, inp)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]
    assert np.array_equal(got["conv_out"].float().cpu().numpy(), ref["conv_out"])


def test_prefill_ragged_many_sequences():
    """Nine packed sequences of the 16/32-head shape: 288 heads, more than the CUs, so the
    carry runs whole-head workgroups (longest sequence first)."""
    shape, dtype = gi.QWEN, "bf16"
    lens = [20, 65, 0, 130, 1, 64, 3, 70, 40]
    cu = gi.cu_seqlens(lens)
    _say(f"prefill ragged, {len(lens)} sequences of the full head shape")
    inp = layer_inputs(shape, 1, int(cu[-1]), 21, dtype, N=len(lens), s0_std=0.1, conv_std=1.0)
    got = run_prefill(shape, dtype, inp, cu=cu)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"], cu_seqlens=cu)
    assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]
    assert np.array_equal(got["conv_out"].float().cpu().numpy(), ref["conv_out"])


@pytest.mark.parametrize("shape,L,cu_given,cu_read", [
    (SMALL128, 260, [-5, 70, 200, 300], [0, 70, 200, 260]),
    (SMALL128, 230, [0, 70, 200, 150, 150], [0, 70, 200, 200, 200]),
    (gi.QWEN, 1050, [0, 900, 1000, 950, 950], [0, 900, 1000, 1000, 1000]),
], ids=["clamped_to_0_and_L", "decreasing_pairs", "decreasing_pairs_full_heads"])
def test_prefill_cu_seqlens_clamped_with_canary(shape, L, cu_given, cu_read):
    """cu_seqlens entries outside [0, L] are clamped and a decreasing pair is an empty
    sequence: the call equals the oracle on the clamped table, the tokens no sequence
    owns keep the NaN o was filled with, and an empty sequence keeps its state bit for
    bit. The last case runs the full head shape, a 15-chunk chain per head split over
    two workgroups."""
    dtype = "bf16"
    N = len(cu_given) - 1
    _say(f"prefill cu_seqlens {cu_given} over L={L}, {shape}")
    inp = layer_inputs(shape, 1, L, 23, dtype, N=N, s0_std=0.1, conv_std=1.0)
    got = run_prefill(shape, dtype, inp, cu=np.asarray(cu_given, np.int32), o_fill=float("nan"))
    n_in = cu_read[-1]
    cut = dict(inp, qkv=inp["qkv"][:, :, :n_in], gate=inp["gate"][:, :n_in],
               beta=inp["beta"][:, :n_in])
    ref = oracle.gdn_forward(oparams(shape), cut["qkv"], cut["gate"], cut["beta"], cut["w"],
                             cut["conv0"], cut["S0"], cu_seqlens=np.asarray(cu_read, np.int32))
    assert bool(torch.isfinite(got["o"][:, :n_in]).all())
    assert rel_err(got["o"][:, :n_in], ref["o"]) <= TOL[dtype]
    assert bool(torch.isnan(got["o"][:, n_in:]).all())
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]
    S0 = torch.from_numpy(inp["S0"])
    for n in range(N):
        if cu_read[n + 1] == cu_read[n]:
            assert torch.equal(got["S"][n].cpu(), S0[n]), f"empty sequence {n} changed its state"
    assert np.array_equal(got["conv_out"].float().cpu().numpy(), ref["conv_out"])


def test_prefill_packed_thousands_of_sequences():
    """5000 packed sequences of 0-3 tokens with a 130-token one every 500: more than the
    front kernel's cu_seqlens table in LDS holds (it then searches the table in memory)
    and more than the carry ranks by length (it then takes them in order). Tokens past
    the last sequence keep the NaN o was filled with; empty sequences keep their state
    bit for bit."""
    shape, dtype = gi.Shape(Hk=1, Hv=2, dk=128, dv=128, K=4), "bf16"
    lens = gi.seq_lens(5000, 0, 3, 24)
    lens[::500] = 130
    cu = gi.cu_seqlens(lens)
    n_in = int(cu[-1])
    L = n_in + 40
    _say(f"prefill, {len(lens)} packed sequences over {n_in} of {L} tokens")
    inp = layer_inputs(shape, 1, L, 24, dtype, N=len(lens), s0_std=0.1, conv_std=1.0)
    got = run_prefill(shape, dtype, inp, cu=cu, o_fill=float("nan"))
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"][:, :, :n_in], inp["gate"][:, :n_in],
                             inp["beta"][:, :n_in], inp["w"], inp["conv0"], inp["S0"], cu_seqlens=cu)
    assert bool(torch.isfinite(got["o"][:, :n_in]).all())
    assert rel_err(got["o"][:, :n_in], ref["o"]) <= TOL[dtype]
    assert bool(torch.isnan(got["o"][:, n_in:]).all())
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]
    empty = torch.from_numpy(np.flatnonzero(lens == 0))
    assert len(empty) > 0
    assert torch.equal(got["S"].cpu()[empty], torch.from_numpy(inp["S0"])[empty])
    assert np.array_equal(got["conv_out"].float().cpu().numpy(), ref["conv_out"])


def test_prefill_packed_cost_grows_linearly_with_sequences():
    """Eight times as many packed sequences (of 4 tokens each) cost about eight times as
    much, not 64 times: no kernel spends time per workgroup on every sequence before its
    own (such a scan made 4,096 sequences cost 24 times what 512 did)."""
    shape, dtype = SMALL128, "bf16"
    p = params(shape, dtype)
    times = {}
    for N in (512, 4096):
        L = 4 * N
        cu = dev(gi.cu_seqlens(np.full(N, 4)))
        inp = layer_inputs(shape, 1, L, 25, dtype, N=N)
        x, g, b, w, c0 = (dev(inp[k], dtype) for k in ("qkv", "gate", "beta", "w", "conv0"))
        c1, S = torch.empty_like(c0), dev(inp["S0"])
        o = torch.empty((1, L, shape.Hv, shape.dv), device="cuda")
        ws = gdn.prefill_workspace(p, 1, L, N)
        call = lambda: gdn.gdn_prefill(p, x, g, b, w, c0, c1, S, o, ws, cu_seqlens=cu)
        for _ in range(2):
            call()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(3):
            call()
        en.record()
        torch.cuda.synchronize()
        times[N] = st.elapsed_time(en) / 3
        _say(f"prefill, {N} packed sequences of 4 tokens: {1e3 * times[N]:.0f} us per call")
    assert times[4096] < 16 * times[512], times


@pytest.mark.parametrize("L,scale", [(512, 0.01), (2000, 0.01), (65536, 0.001)],
                         ids=["one_chain", "eight_segments", "long_context_L65536"])
def test_prefill_long_memory(L, scale):
    """Weak decay (gate scaled by 0.01) so early errors do not fade; beta near 1. At 2000
    tokens the carry runs in 8 segments, whose state maps then stay far from zero and whose
    entry states are chained through up to 6 maps. The 65,536-token prompt (1,024 chunks,
    8 segments of about 130) has its gates scaled by 0.001: a memory of about a thousand
    tokens."""
    shape, dtype = SMALL128, "bf16"
    _say(f"long memory L={L} gate scale {scale}")
    inp = layer_inputs(shape, 1, L, 13, dtype, s0_std=0.1, conv_std=1.0)
    inp["gate"] = gi.round_to(scale * inp["gate"].astype(np.float64), dtype)
    inp["beta"] = gi.round_to(0.5 + 0.5 * inp["beta"].astype(np.float64), dtype)
    got = run_prefill(shape, dtype, inp)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]


@pytest.mark.parametrize("packed", [False, True], ids=["segmented", "one_chain"])
def test_prefill_magnitude_swings(packed):
    """The carry keeps the state's and Delta's power-of-two scales from chunk to chunk and
    moves them only when a value leaves a window of fp16's range. Here the values jump by
    up to 2^40 from one chunk to the next and the decay switches between strong and
    weak, so both scales move in both directions many times; every chunk's outputs must
    still meet the budget against that chunk's own largest output, i.e. keep their relative
    precision at every magnitude. Segmented (pass 1 whole-head, pass 2 half-head
    workgroups) and as one packed sequence (a single chain)."""
    shape, dtype = SMALL128, "bf16"
    L, C = 1300, 64
    _say(f"prefill magnitude swings packed={packed}")
    inp = layer_inputs(shape, 1, L, 23, dtype, s0_std=100.0, conv_std=1.0)
    shifts = [0, 20, -20, 40, -40, 0, 12, -12, 30, -30, 5, -5, 0, 24, -24, 0, 40, 0, -40, 8, 0]
    gates = [1.0, 0.01, 10.0, 0.01, 1.0, 10.0, 0.01, 0.01, 1.0, 10.0, 0.01]
    x = inp["qkv"].astype(np.float64)
    g = inp["gate"].astype(np.float64)
    v0 = 2 * shape.Hk * shape.dk                      # first value channel
    for c in range(0, (L + C - 1) // C):
        sl = slice(c * C, min((c + 1) * C, L))
        x[:, v0:, sl] *= 2.0 ** shifts[c % len(shifts)]
        g[:, sl, :] *= gates[c % len(gates)]
    inp["qkv"] = gi.round_to(x, dtype)                # powers of two: exact in bf16
    inp["gate"] = gi.round_to(g, dtype)
    cu = [0, L] if packed else None
    got = run_prefill(shape, dtype, inp, cu=cu)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"], cu_seqlens=None if cu is None else np.asarray(cu, np.int32))
    o = got["o"].double().cpu().numpy()
    worst = 0.0
    for c in range(0, (L + C - 1) // C):
        sl = slice(c * C, min((c + 1) * C, L))
        worst = max(worst, rel_err(o[:, sl], ref["o"][:, sl]))
    assert worst <= TOL[dtype], worst
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]


@pytest.mark.parametrize("packed", [False, True], ids=["segmented", "one_chain"])
@pytest.mark.parametrize("case", ["no_decay_full_write", "total_forgetting"])
def test_prefill_degenerate_gates(case, packed):
    """The gate's two extremes: g = 0 with beta = 1 (no decay, every write at full strength:
    the state maps never fade and each key's value is recalled exactly after its write),
    and g = -60 per token (the state forgets everything between two tokens: every decay
    factor across a token underflows, the state maps are exactly zero and each output
    depends on its own token only)."""
    shape, dtype, L = SMALL128, "bf16", 1300
    _say(f"prefill degenerate gates {case} packed={packed}")
    inp = layer_inputs(shape, 1, L, 24, dtype, s0_std=0.1, conv_std=1.0)
    if case == "no_decay_full_write":
        inp["gate"] = np.zeros_like(inp["gate"])
        inp["beta"] = gi.round_to(np.ones(inp["beta"].shape), dtype)
    else:
        inp["gate"] = gi.round_to(np.full(inp["gate"].shape, -60.0), dtype)
    cu = [0, L] if packed else None
    got = run_prefill(shape, dtype, inp, cu=cu)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"], cu_seqlens=None if cu is None else np.asarray(cu, np.int32))
    assert not torch.isnan(got["o"]).any()
    assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
    assert rel_err(got["S"], ref["S"]) <= TOL[dtype]


# ---------------------------------------------------------------------------
# decode and verify, small
# ---------------------------------------------------------------------------
def _decode_steps(shape, dtype, inp, steps):
    p = params(shape, dtype)
    B = inp["qkv"].shape[0]
    S = dev(inp["S0"])
    cs = dev(inp["conv0"], dtype)
    w = dev(inp["w"], dtype)
    outs = []
    for t in range(steps):
        o = torch.empty((B, 1, shape.Hv, shape.dv), device="cuda")
        cnew = torch.empty_like(cs)
        gdn.gdn_decode_step(p, dev(inp["qkv"][:, :, t:t + 1], dtype), dev(inp["gate"][:, t:t + 1], dtype),
                            dev(inp["beta"][:, t:t + 1], dtype), w, cs, cnew, S, o)
        cs = cnew
        outs.append(o)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), S, cs


@pytest.mark.parametrize("shape,dtype,B,steps", [(gi.TINY, "f32", 1, 64), (gi.TINY_GQA, "f32", 2, 16),
                                                 (SMALL128, "bf16", 3, 20)])
def test_decode_small(shape, dtype, B, steps):
    _say(f"decode {shape} {dtype} B={B} steps={steps}")
    inp = layer_inputs(shape, B, steps, 21, dtype, s0_std=0.1, conv_std=1.0)
    o, S, cs = _decode_steps(shape, dtype, inp, steps)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cs.float().cpu().numpy(), ref["conv_out"])


@pytest.mark.parametrize("case", ["no_decay_full_write", "total_forgetting"])
def test_decode_and_verify_degenerate_gates(case):
    """The gate's extremes on the recurrent kernel: g = 0 with beta = 1, and g = -60 (the
    carried state is wiped between tokens), as decode steps and as a verify block whose
    snapshots are checked against the oracle's states after each token."""
    shape, dtype, B, steps = SMALL128, "bf16", 3, 12
    _say(f"decode/verify degenerate gates {case}")
    inp = layer_inputs(shape, B, steps, 25, dtype, s0_std=0.5, conv_std=1.0)
    if case == "no_decay_full_write":
        inp["gate"] = np.zeros_like(inp["gate"])
        inp["beta"] = gi.round_to(np.ones(inp["beta"].shape), dtype)
    else:
        inp["gate"] = gi.round_to(np.full(inp["gate"].shape, -60.0), dtype)
    o, S, cs = _decode_steps(shape, dtype, inp, steps)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    T = 4
    blk = {k: (v[:, :, :T] if k == "qkv" else v[:, :T]) if k in ("qkv", "gate", "beta") else v for k, v in inp.items()}
    snap, ov = _verify(shape, dtype, blk, dev(inp["S0"]), dev(inp["conv0"], dtype), T)
    torch.cuda.synchronize()
    for t in range(T):
        r = oracle.gdn_forward(oparams(shape), inp["qkv"][:, :, :t + 1], inp["gate"][:, :t + 1], inp["beta"][:, :t + 1],
                               inp["w"], inp["conv0"], inp["S0"])
        assert rel_err(snap[:, t], r["S"]) <= TOL[dtype], t
        assert rel_err(ov[:, t], r["o"][:, t]) <= TOL[dtype], t


def _verify(shape, dtype, inp, S_in, cs, T):
    p = params(shape, dtype)
    B = inp["qkv"].shape[0]
    snap = torch.empty((B, T, shape.Hv, shape.dk, shape.dv), device="cuda")
    o = torch.empty((B, T, shape.Hv, shape.dv), device="cuda")
    gdn.gdn_verify_block(p, dev(inp["qkv"], dtype), dev(inp["gate"], dtype), dev(inp["beta"], dtype),
                         dev(inp["w"], dtype), cs, S_in, snap, o)
    return snap, o


@pytest.mark.parametrize("shape,dtype,B,blocks,T", [(gi.TINY, "f32", 1, 16, 4), (SMALL128, "bf16", 4, 3, 4),
                                                    (gi.TINY_GQA, "f32", 3, 4, 1), (SMALL128, "bf16", 2, 2, 16)])
def test_verify_commit_chain(shape, dtype, B, blocks, T):
    """Blocks of T tokens; after each, commit a random accepted prefix and carry on
    from it. The oracle replays exactly the committed tokens."""
    _say(f"verify chain {shape} {dtype} B={B} blocks={blocks} T={T}")
    p = params(shape, dtype)
    op = oparams(shape)
    base = layer_inputs(shape, B, 1, 31, dtype, s0_std=0.1, conv_std=1.0)
    S = dev(base["S0"])
    cs = dev(base["conv0"], dtype)
    S_ref = base["S0"].astype(np.float64)
    c_ref = base["conv0"].astype(np.float64)
    for blk in range(blocks):
        inp = layer_inputs(shape, B, T, 31, dtype, step=blk)
        inp["w"] = base["w"]
        snap, o = _verify(shape, dtype, inp, S, cs, T)
        acc = gi.accept_len(B, T, 31 + blk)
        S_new = torch.empty_like(S)
        c_new = torch.empty_like(cs)
        gdn.gdn_verify_commit(p, dev(acc), dev(inp["qkv"], dtype), cs, snap, c_new, S_new)
        torch.cuda.synchronize()
        ref = oracle.gdn_forward(op, inp["qkv"], inp["gate"], inp["beta"], inp["w"], c_ref, S_ref,
                                 snapshots=True)
        assert rel_err(o, ref["o"]) <= TOL[dtype]
        assert rel_err(snap, ref["snap"]) <= TOL[dtype]
        S_ref, c_ref = oracle.verify_commit(op, acc, inp["qkv"], c_ref, ref["snap"])
        assert rel_err(S_new, S_ref) <= TOL[dtype]
        assert np.array_equal(c_new.float().cpu().numpy(), c_ref)
        S, cs = S_new, c_new


@pytest.mark.parametrize("Hk,Hv,dtype", [(4, 16, "f32"), (4, 16, "bf16"), (2, 16, "bf16")],
                         ids=["f4_fp32_path", "f4_mfma_path", "f8_mfma_path"])
def test_gqa_mapping_probe_exact(Hk, Hv, dtype):
    """One token from a zero state, identity conv, beta = 1, gate = 0: o_h = (k.q) v_h
    with k, q from K head h // f. K head j's key makes angle theta_j with its query, so
    round(o_h / v_h) read back as an integer must name h // f for every h, exactly. GQA
    factors 4 and 8, through the fp32 prefill and the MFMA one (bf16 inputs: every probe
    value is exact in bf16)."""
    shape = gi.Shape(Hk=Hk, Hv=Hv, dk=128, dv=128)
    _say(f"GQA probe Hk={Hk} Hv={Hv} {dtype}")
    Hk, Hv, dk, dv, K, D = shape.Hk, shape.Hv, shape.dk, shape.dv, shape.K, shape.D
    x = np.zeros((1, D, 1), np.float32)
    for j in range(Hk):
        x[0, j * dk, 0] = 4.0                    # q of head j along e0
        x[0, Hk * dk + j * dk, 0] = 4.0          # k of head j: direction (1, j+1) scaled
        x[0, Hk * dk + j * dk + 1, 0] = 4.0 * (j + 1)
    x[0, 2 * Hk * dk:, 0] = 1.0                  # v = silu(1) everywhere
    w = np.zeros((D, 1, K), np.float32)
    w[:, 0, K - 1] = 1.0
    p = params(shape, dtype)
    inp = {"qkv": x, "gate": np.zeros((1, 1, Hv), np.float32), "beta": np.ones((1, 1, Hv), np.float32),
           "w": w, "conv0": np.zeros((1, D, K - 1), np.float32), "S0": np.zeros((1, Hv, dk, dv), np.float32)}
    got = run_prefill(shape, dtype, inp)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    silu1 = 1.0 / (1.0 + np.exp(-1.0))
    # (k.q) sqrt(dk) = cos(theta_j) identifies head j; map it back to j
    cos = got["o"][0, 0, :, 0].double().cpu().numpy() * np.sqrt(dk) / silu1
    cos_ref = ref["o"][0, 0, :, 0] * np.sqrt(dk) / silu1

    def head_of(c):
        # silu(4 (j+1)) / silu(4) ~ (j+1): the k direction is (1, ~j+1) up to SiLU
        return np.rint(np.sqrt(np.maximum(1.0 / np.maximum(c, 1e-9) ** 2 - 1.0, 0.0)) - 1.0).astype(int)
    assert np.array_equal(head_of(cos), np.arange(Hv) // (Hv // Hk))
    assert np.array_equal(head_of(cos), head_of(cos_ref))
    # decode and verify use their own indexing: same probe through both
    o_dec = torch.empty((1, 1, Hv, dv), device="cuda")
    S = torch.zeros((1, Hv, dk, dv), device="cuda")
    cz = dev(inp["conv0"], dtype)
    gdn.gdn_decode_step(p, dev(x, dtype), dev(inp["gate"], dtype), dev(inp["beta"], dtype), dev(w, dtype), cz,
                        torch.empty_like(cz), S, o_dec)
    torch.cuda.synchronize()
    assert np.array_equal(head_of(o_dec[0, 0, :, 0].double().cpu().numpy() * np.sqrt(dk) / silu1),
                          np.arange(Hv) // (Hv // Hk))


# ---------------------------------------------------------------------------
# bit-exact GPU invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 6, 16])
def test_verify_snapshots_equal_decode_steps_bitexact(T):
    """A verify block of width T (1: the decode layout; 6 and 16, the widest: the narrow
    layout) gives the decode steps' outputs and states bit for bit."""
    shape, dtype, B = SMALL128, "bf16", 5
    inp = layer_inputs(shape, B, T, 41, dtype, s0_std=0.1, conv_std=1.0)
    S0 = dev(inp["S0"])
    snap, o_v = _verify(shape, dtype, inp, S0, dev(inp["conv0"], dtype), T)
    o_d, S_d, _ = _decode_steps(shape, dtype, inp, T)
    torch.cuda.synchronize()
    assert torch.equal(o_v, o_d)
    assert torch.equal(snap[:, -1], S_d)
    # every intermediate snapshot too
    S = dev(inp["S0"])
    cs = dev(inp["conv0"], dtype)
    p = params(shape, dtype)
    for t in range(T):
        o = torch.empty((B, 1, shape.Hv, shape.dv), device="cuda")
        cn = torch.empty_like(cs)
        gdn.gdn_decode_step(p, dev(inp["qkv"][:, :, t:t + 1], dtype), dev(inp["gate"][:, t:t + 1], dtype),
                            dev(inp["beta"][:, t:t + 1], dtype), dev(inp["w"], dtype), cs, cn, S, o)
        cs = cn
        torch.cuda.synchronize()
        assert torch.equal(snap[:, t], S)


def test_beta0_gate0_keeps_state_bitexact():
    shape, dtype, B = SMALL128, "bf16", 3
    inp = layer_inputs(shape, B, 1, 42, dtype, s0_std=0.1, conv_std=1.0)
    p = params(shape, dtype)
    S = dev(inp["S0"])
    S_before = S.clone()
    o = torch.empty((B, 1, shape.Hv, shape.dv), device="cuda")
    z = torch.zeros((B, 1, shape.Hv), device="cuda", dtype=torch.bfloat16)
    cs = dev(inp["conv0"], dtype)
    gdn.gdn_decode_step(p, dev(inp["qkv"], dtype), z, z, dev(inp["w"], dtype), cs, torch.empty_like(cs), S, o)
    torch.cuda.synchronize()
    assert torch.equal(S, S_before)
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], np.zeros((B, 1, shape.Hv)), np.zeros((B, 1, shape.Hv)),
                             inp["w"], inp["conv0"], inp["S0"])
    assert rel_err(o, ref["o"]) <= TOL[dtype]


def test_prefill_deterministic_and_ragged_equals_separate():
    shape, dtype = SMALL128, "bf16"
    lens = [100, 3, 64, 0, 65]
    cu = gi.cu_seqlens(lens)
    inp = layer_inputs(shape, 1, int(cu[-1]), 43, dtype, N=len(lens), s0_std=0.1, conv_std=1.0)
    a = run_prefill(shape, dtype, inp, cu=cu)
    b = run_prefill(shape, dtype, inp, cu=cu)
    for k in ("o", "S", "conv_out"):
        assert torch.equal(a[k], b[k]), k
    # Each sequence alone, through cu_seqlens = [0, len] and unpacked: every (chunk, head)
    # and every carry workgroup does the same arithmetic whatever else is packed beside it
    # (chains this short never run in segments), so the results agree bit for bit.
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        one = {"qkv": inp["qkv"][:, :, s:e], "gate": inp["gate"][:, s:e], "beta": inp["beta"][:, s:e],
               "w": inp["w"], "conv0": inp["conv0"][n:n + 1], "S0": inp["S0"][n:n + 1]}
        for r in (run_prefill(shape, dtype, one, cu=gi.cu_seqlens([e - s])), run_prefill(shape, dtype, one)):
            assert torch.equal(r["conv_out"][0], a["conv_out"][n]), n
            assert torch.equal(r["o"][0], a["o"][0, s:e]), n
            assert torch.equal(r["S"][0], a["S"][n]), n


@pytest.mark.parametrize("L", [65, 700, 768, 1000, 1300, 2000])
def test_prefill_segmented_carry(L):
    """A lone prompt of 4 heads runs the carry in segments once it has 12 chunks or more
    (3 segments at 768 tokens, 4 at 1000 with a ragged last chunk, 5 at 1300, 8 at 2000;
    one chain below that); the packed path (one sequence through cu_seqlens) never
    does. Both agree with the oracle."""
    shape, dtype = SMALL128, "bf16"
    _say(f"segmented carry L={L}")
    inp = layer_inputs(shape, 1, L, 45, dtype, s0_std=0.1, conv_std=1.0)
    seg = run_prefill(shape, dtype, inp)
    packed = run_prefill(shape, dtype, inp, cu=gi.cu_seqlens([L]))
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    for got in (seg, packed):
        assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
        assert rel_err(got["S"], ref["S"]) <= TOL[dtype]
        assert np.array_equal(got["conv_out"].float().cpu().numpy(), ref["conv_out"])


@pytest.mark.parametrize("L", [1300, 2000])
def test_prefill_segmented_zero_column_map(L):
    """Segment state maps whose first column is exactly zero while the rest of its 16-column
    tile is not. Every key is the unit vector e_0 (K channel 0 of each head constant, every
    other K channel zero, identity conv taps), beta = 1 and gate = 0, so each token replaces
    row 0 of S by its value and leaves the other rows alone: a segment's map is I - e_0 e_0^T.
    The tile of map columns 0..15 must keep its scale (a zero-tile flag taken from one lane
    would drop rows 1..15 of every later entry state). 5 and 8 segments."""
    shape, dtype = SMALL128, "bf16"
    _say(f"segmented carry, zero map column L={L}")
    rng = np.random.default_rng([1301, L])
    D, HKD = shape.D, shape.Hk * shape.dk
    x = np.zeros((1, D, L))
    x[:, :HKD] = rng.standard_normal((1, HKD, L))                 # queries
    x[:, 2 * HKD:] = rng.standard_normal((1, D - 2 * HKD, L))      # values
    for hk in range(shape.Hk):
        x[:, HKD + hk * shape.dk] = 4.0                            # key channel 0 of head hk
    w = np.zeros((D, 1, shape.K))
    w[:, 0, shape.K - 1] = 1.0                                     # conv = current token
    inp = {"qkv": gi.round_to(x, dtype), "gate": np.zeros((1, L, shape.Hv), np.float32),
           "beta": np.ones((1, L, shape.Hv), np.float32), "w": gi.round_to(w, dtype),
           "conv0": np.zeros((1, D, shape.K - 1), np.float32), "S0": gi.state0(shape, 1, 47, 0.1)}
    seg = run_prefill(shape, dtype, inp)
    packed = run_prefill(shape, dtype, inp, cu=gi.cu_seqlens([L]))
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    for got in (seg, packed):
        assert rel_err(got["o"], ref["o"]) <= TOL[dtype]
        assert rel_err(got["S"], ref["S"]) <= TOL[dtype]


@pytest.mark.parametrize("B,L", [(1, 768), (2, 800), (1, 2000)])
def test_prefill_front_paths_bitexact(B, L):
    """The front kernel's interior tiles take a 16-byte vector path when the rows are bf16,
    unpacked, a multiple of 8 tokens long and qkv is 16-byte aligned; with qkv one element
    off that alignment every tile takes the general path. Both do the same arithmetic in the
    same order, so the whole layer agrees bit for bit (and with the oracle)."""
    shape, dtype = SMALL128, "bf16"
    _say(f"front paths B={B} L={L}")
    inp = layer_inputs(shape, B, L, 46, dtype, s0_std=0.1, conv_std=1.0)
    vec = run_prefill(shape, dtype, inp)
    gen = run_prefill(shape, dtype, inp, qkv_offset=1)
    for k in ("o", "S", "conv_out"):
        assert torch.equal(vec[k], gen[k]), k
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(vec["o"], ref["o"]) <= TOL[dtype]
    assert rel_err(vec["S"], ref["S"]) <= TOL[dtype]


def test_prefill_split_carry():
    """prefill(L) == prefill(L1) then prefill(L - L1) with both states carried."""
    shape, dtype = SMALL128, "bf16"
    inp = layer_inputs(shape, 1, 300, 44, dtype, s0_std=0.1, conv_std=1.0)
    full = run_prefill(shape, dtype, inp)
    first = {k: v for k, v in inp.items()}
    first.update(qkv=inp["qkv"][:, :, :77], gate=inp["gate"][:, :77], beta=inp["beta"][:, :77])
    r1 = run_prefill(shape, dtype, first)
    second = {"qkv": inp["qkv"][:, :, 77:], "gate": inp["gate"][:, 77:], "beta": inp["beta"][:, 77:],
              "w": inp["w"], "conv0": r1["conv_out"].float().cpu().numpy(), "S0": r1["S"].cpu().numpy()}
    r2 = run_prefill(shape, dtype, second)
    ref_o = full["o"].double().cpu().numpy()
    assert rel_err(torch.cat([r1["o"], r2["o"]], dim=1), ref_o) <= TOL[dtype]
    assert rel_err(r2["S"], full["S"].double().cpu().numpy()) <= TOL[dtype]
    assert torch.equal(r2["conv_out"], full["conv_out"])


def test_empty_calls_launch_nothing():
    shape, dtype = SMALL128, "bf16"
    p = params(shape, dtype)
    inp = layer_inputs(shape, 1, 0, 45, dtype, s0_std=0.1)
    got = run_prefill(shape, dtype, inp)   # L = 0: S and the conv window come back unchanged
    assert torch.equal(got["S"].cpu(), torch.from_numpy(inp["S0"]))
    assert torch.equal(got["conv_out"].float().cpu(), torch.from_numpy(inp["conv0"]))
    e = torch.empty(0, device="cuda")
    gdn.gdn_decode_step(p, e.reshape(0, shape.D, 1).bfloat16(), e.reshape(0, 1, 4).bfloat16(),
                        e.reshape(0, 1, 4).bfloat16(), torch.zeros((shape.D, 1, 4), device="cuda").bfloat16(),
                        e.reshape(0, shape.D, 3).bfloat16(), e.reshape(0, shape.D, 3).bfloat16(),
                        e.reshape(0, 4, 128, 128), e.reshape(0, 1, 4, 128))


def test_calls_never_synchronise():
    """Enqueue a long chain of matmuls, then the library calls: each must return
    while the chain is still running (it only enqueues)."""
    shape, dtype, B = SMALL128, "bf16", 4
    inp = layer_inputs(shape, B, 64, 46, dtype, s0_std=0.1, conv_std=1.0)
    p = params(shape, dtype)
    args = {k: dev(v, dtype if k not in ("S0",) else None) for k, v in inp.items()}
    ws = gdn.prefill_workspace(p, B, 64, B)
    o = torch.empty((B, 64, shape.Hv, shape.dv), device="cuda")
    cout = torch.empty_like(args["conv0"])
    snap = torch.empty((B, 4, shape.Hv, 128, 128), device="cuda")
    a = torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    for _ in range(60):
        a = a @ a
        a = a / a.norm()
    t0 = time.perf_counter()
    gdn.gdn_prefill(p, args["qkv"], args["gate"], args["beta"], args["w"], args["conv0"], cout,
                    args["S0"], o, ws)
    gdn.gdn_verify_block(p, args["qkv"][:, :, :4].contiguous(), args["gate"][:, :4].contiguous(),
                         args["beta"][:, :4].contiguous(), args["w"], args["conv0"], args["S0"], snap,
                         o[:, :4].contiguous())
    t1 = time.perf_counter()
    pending = not torch.cuda.current_stream().query()
    torch.cuda.synchronize()
    assert pending, "the matmul chain drained before the library calls returned"
    assert t1 - t0 < 0.05
