"""GPU parity of the layer variants: no L2 norm of q and k (use_qk_l2norm = 0),
no GQA (Hv == Hk), fp32 inputs at d = 128, and head dim 64, on decode, verify
(with commit) and prefill (plain and packed), against the fp64 oracle on the
same seeded inputs. Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_sequence_amd as gdn
import oracle
from gpu_cases import TOL, dev, layer_inputs, oparams, params, rel_err

pytestmark = pytest.mark.gpu

D64 = gi.Shape(Hk=2, Hv=4, dk=64, dv=64, K=4)
NOGQA128 = gi.Shape(Hk=4, Hv=4, dk=128, dv=128, K=4)
NOGQA16 = gi.Shape(Hk=3, Hv=3, dk=16, dv=16, K=4)
SMALL128 = gi.Shape(Hk=2, Hv=4, dk=128, dv=128, K=4)
GQA8 = gi.Shape(Hk=2, Hv=16, dk=128, dv=128, K=4)   # eight V heads per K head

# (shape, input dtype, use_qk_l2norm)
VARIANTS = [
    (D64, "bf16", True), (D64, "f32", True), (D64, "bf16", False),
    (NOGQA128, "bf16", True), (NOGQA128, "f32", True), (NOGQA16, "f32", True),
    (SMALL128, "bf16", False), (SMALL128, "f32", False), (gi.TINY_GQA, "f32", False),
    (GQA8, "bf16", True),
]
IDS = [f"{s.Hk}x{s.Hv}_d{s.dk}_{dt}_{'l2' if l2 else 'nol2'}" for s, dt, l2 in VARIANTS]


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    oracle.build_oracle(force=False)


def _inputs(shape, B, L, seed, dtype, use_l2, N=None, step=None):
    """Seeded inputs; without the L2 norm the qkv columns are scaled by 0.15 (and
    re-rounded) so that |k|^2 stays near 1 and the recurrence stays contractive."""
    inp = layer_inputs(shape, B, L, seed, dtype, N=N, s0_std=0.1, conv_std=1.0, step=step)
    if not use_l2:
        inp["qkv"] = gi.round_to(0.15 * inp["qkv"].astype(np.float64), dtype)
        inp["conv0"] = gi.round_to(0.15 * inp["conv0"].astype(np.float64), dtype)
    return inp


@pytest.mark.parametrize("shape,dtype,use_l2", VARIANTS, ids=IDS)
def test_decode_variant(shape, dtype, use_l2):
    print(f"decode variant {shape} {dtype} l2={use_l2}", flush=True)
    B, steps = 2, 6
    p, op = params(shape, dtype, use_l2), oparams(shape, use_l2)
    inp = _inputs(shape, B, steps, 71, dtype, use_l2)
    S, cs, w = dev(inp["S0"]), dev(inp["conv0"], dtype), dev(inp["w"], dtype)
    outs = []
    for t in range(steps):
        o = torch.empty((B, 1, shape.Hv, shape.dv), device="cuda")
        cn = torch.empty_like(cs)
        gdn.gdn_decode_step(p, dev(inp["qkv"][:, :, t:t + 1], dtype), dev(inp["gate"][:, t:t + 1], dtype),
                            dev(inp["beta"][:, t:t + 1], dtype), w, cs, cn, S, o)
        cs = cn
        outs.append(o)
    torch.cuda.synchronize()
    ref = oracle.gdn_forward(op, inp["qkv"], inp["gate"], inp["beta"], inp["w"], inp["conv0"], inp["S0"])
    assert rel_err(torch.cat(outs, 1), ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cs.float().cpu().numpy(), ref["conv_out"])


@pytest.mark.parametrize("shape,dtype,use_l2", VARIANTS, ids=IDS)
def test_verify_commit_variant(shape, dtype, use_l2):
    print(f"verify variant {shape} {dtype} l2={use_l2}", flush=True)
    B, T = 3, 4
    p, op = params(shape, dtype, use_l2), oparams(shape, use_l2)
    inp = _inputs(shape, B, T, 72, dtype, use_l2)
    snap = torch.empty((B, T, shape.Hv, shape.dk, shape.dv), device="cuda")
    o = torch.empty((B, T, shape.Hv, shape.dv), device="cuda")
    x, cs = dev(inp["qkv"], dtype), dev(inp["conv0"], dtype)
    gdn.gdn_verify_block(p, x, dev(inp["gate"], dtype), dev(inp["beta"], dtype), dev(inp["w"], dtype),
                         cs, dev(inp["S0"]), snap, o)
    acc = gi.accept_len(B, T, 72)
    S_out, c_out = torch.empty((B, shape.Hv, shape.dk, shape.dv), device="cuda"), torch.empty_like(cs)
    gdn.gdn_verify_commit(p, dev(acc), x, cs, snap, c_out, S_out)
    torch.cuda.synchronize()
    ref = oracle.gdn_forward(op, inp["qkv"], inp["gate"], inp["beta"], inp["w"], inp["conv0"], inp["S0"],
                             snapshots=True)
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(snap, ref["snap"]) <= TOL[dtype]
    S_ref, c_ref = oracle.verify_commit(op, acc, inp["qkv"], inp["conv0"], ref["snap"])
    assert rel_err(S_out, S_ref) <= TOL[dtype]
    assert np.array_equal(c_out.float().cpu().numpy(), c_ref)


def _prefill(shape, dtype, use_l2, inp, cu=None):
    p = params(shape, dtype, use_l2)
    B, _, L = inp["qkv"].shape
    N = inp["S0"].shape[0]
    S = dev(inp["S0"])
    o = torch.zeros((B, L, shape.Hv, shape.dv), device="cuda")
    cout = torch.zeros_like(dev(inp["conv0"], dtype))
    ws = gdn.prefill_workspace(p, B, L, N)
    gdn.gdn_prefill(p, dev(inp["qkv"], dtype), dev(inp["gate"], dtype), dev(inp["beta"], dtype),
                    dev(inp["w"], dtype), dev(inp["conv0"], dtype), cout, S, o, ws,
                    cu_seqlens=None if cu is None else dev(np.asarray(cu, np.int32)))
    torch.cuda.synchronize()
    return o, S, cout


@pytest.mark.parametrize("shape,dtype,use_l2", VARIANTS, ids=IDS)
def test_prefill_variant(shape, dtype, use_l2):
    print(f"prefill variant {shape} {dtype} l2={use_l2}", flush=True)
    inp = _inputs(shape, 2, 150, 73, dtype, use_l2)
    o, S, cout = _prefill(shape, dtype, use_l2, inp)
    ref = oracle.gdn_forward(oparams(shape, use_l2), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


@pytest.mark.parametrize("shape,dtype,use_l2", [(D64, "bf16", True), (NOGQA128, "bf16", True),
                                                 (SMALL128, "bf16", False), (GQA8, "bf16", True)],
                         ids=["d64", "nogqa128", "nol2_128", "gqa8"])
def test_prefill_ragged_variant(shape, dtype, use_l2):
    lens = [70, 0, 130, 1, 64]
    cu = gi.cu_seqlens(lens)
    inp = _inputs(shape, 1, int(cu[-1]), 74, dtype, use_l2, N=len(lens))
    o, S, cout = _prefill(shape, dtype, use_l2, inp, cu=cu)
    ref = oracle.gdn_forward(oparams(shape, use_l2), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"], cu_seqlens=cu)
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def test_prefill_gqa8_segmented():
    """Eight V heads per K head on the MFMA path, one 1,300-token prompt: 16 heads, so the
    carry runs in 5 segments."""
    shape, dtype = GQA8, "bf16"
    print("prefill GQA 8, segmented", flush=True)
    inp = _inputs(shape, 1, 1300, 75, dtype, True)
    o, S, cout = _prefill(shape, dtype, True, inp)
    ref = oracle.gdn_forward(oparams(shape, True), inp["qkv"], inp["gate"], inp["beta"], inp["w"],
                             inp["conv0"], inp["S0"])
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])
