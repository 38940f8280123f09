"""GPU parity of speculative verify at block widths 2..8 and of the zero-copy
chain: the next block starts from the previous block's snapshot slot
(gdn_verify_block_slots, snapshots updated in place) after a window-only commit,
instead of copying the accepted state. Checked against the fp64 oracle's
replay of the committed tokens, and bit for bit against the copying chain.
Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_sequence_amd as gdn
import oracle
from gpu_cases import TOL, dev, layer_inputs, oparams, params, rel_err

pytestmark = pytest.mark.gpu

SMALL128 = gi.Shape(Hk=2, Hv=4, dk=128, dv=128, K=4)


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    oracle.build_oracle(force=False)


def _say(msg):
    print(msg, flush=True)


def _block(shape, dtype, B, T, blk, base):
    inp = layer_inputs(shape, B, T, 61, dtype, step=blk)
    inp["w"] = base["w"]
    return inp


def _run_chain(shape, dtype, B, widths, accept=None):
    """Run the copying chain and the zero-copy chain side by side over blocks of the
    given widths; check both against the oracle and against each other. accept(blk, T)
    gives the accepted lengths of a block (default: drawn uniformly from 0..T-1)."""
    p = params(shape, dtype)
    op = oparams(shape)
    base = layer_inputs(shape, B, 1, 61, dtype, s0_std=0.1, conv_std=1.0)
    w = dev(base["w"], dtype)
    # copying chain
    S_a, cs_a = dev(base["S0"]), dev(base["conv0"], dtype)
    # zero-copy chain: snapshots of the previous block plus its accept lengths
    cs_b = dev(base["conv0"], dtype)
    snap_b, acc_prev = None, None
    S_ref, c_ref = base["S0"].astype(np.float64), base["conv0"].astype(np.float64)
    for blk, T in enumerate(widths):
        inp = _block(shape, dtype, B, T, blk, base)
        x, g, b = dev(inp["qkv"], dtype), dev(inp["gate"], dtype), dev(inp["beta"], dtype)
        snap_a = torch.empty((B, T, shape.Hv, shape.dk, shape.dv), device="cuda")
        o_a = torch.empty((B, T, shape.Hv, shape.dv), device="cuda")
        gdn.gdn_verify_block(p, x, g, b, w, cs_a, S_a, snap_a, o_a)
        o_b = torch.empty_like(o_a)
        if snap_b is None:
            snap_b = torch.empty_like(snap_a)
            gdn.gdn_verify_block(p, x, g, b, w, cs_b, dev(base["S0"]), snap_b, o_b)
        elif snap_b.shape[1] == T:      # same width: snapshots updated in place
            gdn.gdn_verify_block_slots(p, None, x, g, b, w, cs_b, snap_b, acc_prev, snap_b, o_b)
        else:                           # width changes: a fresh snapshot buffer
            nxt = torch.empty_like(snap_a)
            gdn.gdn_verify_block_slots(p, None, x, g, b, w, cs_b, snap_b, acc_prev, nxt, o_b)
            snap_b = nxt
        acc = gi.accept_len(B, T, 61 + blk) if accept is None else accept(blk, T)
        acc_d = dev(acc)
        S_new, c_new = torch.empty_like(S_a), torch.empty_like(cs_a)
        gdn.gdn_verify_commit(p, acc_d, x, cs_a, snap_a, c_new, S_new)
        c_new_b = torch.empty_like(cs_b)
        gdn.gdn_verify_commit(p, acc_d, x, cs_b, None, c_new_b, None)
        torch.cuda.synchronize()
        ref = oracle.gdn_forward(op, inp["qkv"], inp["gate"], inp["beta"], inp["w"], c_ref, S_ref,
                                 snapshots=True)
        assert rel_err(o_a, ref["o"]) <= TOL[dtype]
        assert rel_err(snap_a, ref["snap"]) <= TOL[dtype]
        assert torch.equal(o_a, o_b), f"block {blk}: outputs differ between the chains"
        assert torch.equal(snap_a, snap_b), f"block {blk}: snapshots differ between the chains"
        S_ref, c_ref = oracle.verify_commit(op, acc, inp["qkv"], c_ref, ref["snap"])
        assert rel_err(S_new, S_ref) <= TOL[dtype]
        assert np.array_equal(c_new.float().cpu().numpy(), c_ref)
        assert torch.equal(c_new, c_new_b)
        S_a, cs_a, cs_b, acc_prev = S_new, c_new, c_new_b, acc_d


@pytest.mark.parametrize("T", [2, 3, 4, 5, 6, 7, 8])
def test_verify_width_zero_copy_chain(T):
    _say(f"verify width {T}, zero-copy chain, SMALL128 bf16")
    _run_chain(SMALL128, "bf16", 3, [T, T, T])


@pytest.mark.parametrize("T", [2, 8])
def test_verify_width_tiny_f32(T):
    _say(f"verify width {T}, zero-copy chain, tiny fp32")
    _run_chain(gi.TINY_GQA, "f32", 2, [T, T, T, T])


@pytest.mark.parametrize("T", [2, 16])
def test_verify_accept_extremes(T):
    """Every block accepts nothing for some rows (length 0: the state after the first
    token) and everything for others (length T-1), rotating over the rows."""
    _say(f"verify width {T}, accept lengths 0 and T-1")
    pattern = np.array([0, T - 1, T - 1, 0], np.int32)
    _run_chain(SMALL128, "bf16", 4, [T, T, T, T], accept=lambda blk, T: np.roll(pattern, blk))


def test_verify_commit_clamps_accept_len():
    """accept_len outside [0, T-1] is clamped: the commit equals the one with the
    clamped lengths, bit for bit, for the state and the conv window."""
    shape, dtype, B, T = SMALL128, "bf16", 4, 3
    p = params(shape, dtype)
    inp = layer_inputs(shape, B, T, 64, dtype, s0_std=0.1, conv_std=1.0)
    x, g, b, w, cs = (dev(inp[k], dtype) for k in ("qkv", "gate", "beta", "w", "conv0"))
    snap = torch.empty((B, T, shape.Hv, shape.dk, shape.dv), device="cuda")
    o = torch.empty((B, T, shape.Hv, shape.dv), device="cuda")
    gdn.gdn_verify_block(p, x, g, b, w, cs, dev(inp["S0"]), snap, o)
    outs = []
    for acc in ([-3, 0, 2, 9], [0, 0, 2, 2]):
        S_new, c_new = torch.full_like(snap[:, 0], float("nan")), torch.empty_like(cs)
        gdn.gdn_verify_commit(p, dev(np.array(acc, np.int32)), x, cs, snap, c_new, S_new)
        outs.append((S_new, c_new))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[1][0], snap[torch.arange(B), torch.tensor([0, 0, 2, 2])])


def test_verify_mixed_widths():
    """Block widths change from block to block (snapshots of width T_prev feed a
    block of width T)."""
    _say("verify widths 3, 5, 5, 2, 8")
    _run_chain(SMALL128, "bf16", 2, [3, 5, 5, 2, 8])


def test_verify_slots_with_fusion_bitexact():
    """With the gate/beta prologue and gated-RMSNorm epilogue, starting from slots
    equals starting from the copied state, bit for bit."""
    shape, dtype, B, T = SMALL128, "bf16", 3, 4
    p = params(shape, dtype)
    inp = layer_inputs(shape, B, T, 62, dtype, s0_std=0.1, conv_std=1.0)
    fu = gdn.GdnFusion(dev(gi.a_log(shape, 62, dtype), dtype), dev(gi.dt_bias(shape, 62, dtype), dtype),
                       dev(gi.z_gate(shape, B, T, 62, dtype), dtype), dev(gi.norm_weight(shape, 62, dtype), dtype),
                       1e-6)
    a = dev(gi.a_raw(shape, B, T, 62, dtype), dtype)
    b = dev(gi.b_raw(shape, B, T, 62, dtype), dtype)
    x, w, cs = dev(inp["qkv"], dtype), dev(inp["w"], dtype), dev(inp["conv0"], dtype)
    prev = torch.randn((B, 5, shape.Hv, shape.dk, shape.dv), device="cuda") * 0.1
    slot = dev(np.array([4, 0, 2], np.int32))
    S_in = torch.stack([prev[i, int(k)] for i, k in enumerate([4, 0, 2])]).contiguous()
    snap1, o1 = torch.empty((B, T, shape.Hv, shape.dk, shape.dv), device="cuda"), torch.empty((B, T, shape.Hv, shape.dv), device="cuda")
    snap2, o2 = torch.empty_like(snap1), torch.empty_like(o1)
    gdn.gdn_verify_block_ex(p, fu, x, a, b, w, cs, S_in, snap1, o1)
    gdn.gdn_verify_block_slots(p, fu, x, a, b, w, cs, prev, slot, snap2, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(snap1, snap2)


def test_verify_slots_clamps_slot():
    """Out-of-range slots are clamped into [0, T_prev - 1]."""
    shape, dtype, B, T = gi.TINY, "f32", 3, 2
    p = params(shape, dtype)
    inp = layer_inputs(shape, B, T, 63, dtype, s0_std=0.1, conv_std=1.0)
    x, g, b, w, cs = (dev(inp[k], dtype) for k in ("qkv", "gate", "beta", "w", "conv0"))
    prev = torch.randn((B, 3, shape.Hv, shape.dk, shape.dv), device="cuda")
    slot = dev(np.array([-5, 7, 1], np.int32))
    S_in = torch.stack([prev[0, 0], prev[1, 2], prev[2, 1]]).contiguous()
    snap1, o1 = torch.empty((B, T, shape.Hv, shape.dk, shape.dv), device="cuda"), torch.empty((B, T, shape.Hv, shape.dv), device="cuda")
    snap2, o2 = torch.empty_like(snap1), torch.empty_like(o1)
    gdn.gdn_verify_block(p, x, g, b, w, cs, S_in, snap1, o1)
    gdn.gdn_verify_block_slots(p, None, x, g, b, w, cs, prev, slot, snap2, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(snap1, snap2)
