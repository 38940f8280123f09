"""GPU parity of the optional fusions of gdn_fusion (the *_ex entry points):
the gate/beta prologue and the gated-RMSNorm epilogue, each alone and together,
on the decode, verify and prefill paths (fp32 vector and fp16-MFMA prefill),
against oracle.gate_beta -> oracle.gdn_forward -> oracle.gated_rmsnorm on the
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

SMALL128 = gi.Shape(Hk=2, Hv=4, dk=128, dv=128, K=4)
EPS = 1e-6


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    oracle.build_oracle(force=False)


def _say(msg):
    print(msg, flush=True)


def fused_inputs(shape, B, L, seed, dtype, pro, epi, N=None, s0=0.1):
    """layer_inputs plus the fusion tensors. With the prologue, gate/beta are
    replaced by the raw projections; the oracle's gate/beta are derived from
    them by oracle.gate_beta."""
    inp = layer_inputs(shape, B, L, seed, dtype, N=N, s0_std=s0, conv_std=1.0)
    if pro:
        inp["a"] = gi.a_raw(shape, B, L, seed, dtype)
        inp["b"] = gi.b_raw(shape, B, L, seed, dtype)
        inp["A_log"] = gi.a_log(shape, seed, dtype)
        inp["dt_bias"] = gi.dt_bias(shape, seed, dtype)
    if epi:
        inp["z"] = gi.z_gate(shape, B, L, seed, dtype)
        inp["norm_w"] = gi.norm_weight(shape, seed, dtype)
    return inp


def fusion_of(inp, dtype, t=None):
    """GdnFusion of device tensors (z sliced to token t when given)."""
    f = gdn.GdnFusion(norm_eps=EPS)
    if "A_log" in inp:
        f.A_log, f.dt_bias = dev(inp["A_log"], dtype), dev(inp["dt_bias"], dtype)
    if "z" in inp:
        z = inp["z"] if t is None else inp["z"][:, t:t + 1]
        f.z, f.norm_weight = dev(z, dtype), dev(inp["norm_w"], dtype)
    return f


def gate_inputs(inp):
    """What the kernels receive in the gate/beta slots."""
    return (inp["a"], inp["b"]) if "A_log" in inp else (inp["gate"], inp["beta"])


def reference(shape, inp, cu=None):
    if "A_log" in inp:
        g, b = oracle.gate_beta(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    else:
        g, b = inp["gate"], inp["beta"]
    ref = oracle.gdn_forward(oparams(shape), inp["qkv"], g, b, inp["w"], inp["conv0"], inp["S0"],
                             cu_seqlens=cu)
    if "z" in inp:
        ref["o"] = oracle.gated_rmsnorm(ref["o"], inp["z"], inp["norm_w"], EPS)
    return ref


def run_decode(shape, dtype, inp, steps):
    p = params(shape, dtype)
    B = inp["qkv"].shape[0]
    S, cs, w = dev(inp["S0"]), dev(inp["conv0"], dtype), dev(inp["w"], dtype)
    ga, be = gate_inputs(inp)
    outs = []
    for t in range(steps):
        o = torch.empty((B, 1, shape.Hv, shape.dv), device="cuda")
        cn = torch.empty_like(cs)
        gdn.gdn_decode_step_ex(p, fusion_of(inp, dtype, t), dev(inp["qkv"][:, :, t:t + 1], dtype),
                               dev(ga[:, t:t + 1], dtype), dev(be[:, t:t + 1], dtype), w, cs, cn, S, o)
        cs = cn
        outs.append(o)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), S, cs


def run_verify(shape, dtype, inp, T):
    p = params(shape, dtype)
    B = inp["qkv"].shape[0]
    ga, be = gate_inputs(inp)
    snap = torch.empty((B, T, shape.Hv, shape.dk, shape.dv), device="cuda")
    o = torch.empty((B, T, shape.Hv, shape.dv), device="cuda")
    gdn.gdn_verify_block_ex(p, fusion_of(inp, dtype), dev(inp["qkv"], dtype), dev(ga, dtype),
                            dev(be, dtype), dev(inp["w"], dtype), dev(inp["conv0"], dtype),
                            dev(inp["S0"]), snap, o)
    torch.cuda.synchronize()
    return o, snap


def run_prefill(shape, dtype, inp, cu=None, o_fill=0.0):
    p = params(shape, dtype)
    B, _, L = inp["qkv"].shape
    N = inp["S0"].shape[0]
    ga, be = gate_inputs(inp)
    S = dev(inp["S0"])
    o = torch.full((B, L, shape.Hv, shape.dv), o_fill, dtype=torch.float32, device="cuda")
    cout = torch.zeros_like(dev(inp["conv0"], dtype))
    ws = gdn.prefill_workspace(p, B, L, N)
    gdn.gdn_prefill_ex(p, fusion_of(inp, dtype), dev(inp["qkv"], dtype), dev(ga, dtype),
                       dev(be, dtype), dev(inp["w"], dtype), dev(inp["conv0"], dtype), cout, S, o,
                       ws, cu_seqlens=None if cu is None else dev(np.asarray(cu, np.int32)))
    torch.cuda.synchronize()
    return o, S, cout


FUSIONS = [(True, False), (False, True), (True, True)]


@pytest.mark.parametrize("pro,epi", FUSIONS)
@pytest.mark.parametrize("shape,dtype,B,steps", [(gi.TINY_GQA, "f32", 2, 12), (SMALL128, "bf16", 3, 10),
                                                 (SMALL128, "f32", 2, 6)])
def test_decode_fused(shape, dtype, B, steps, pro, epi):
    _say(f"decode_ex {shape} {dtype} B={B} steps={steps} prologue={pro} epilogue={epi}")
    inp = fused_inputs(shape, B, steps, 51, dtype, pro, epi)
    o, S, cs = run_decode(shape, dtype, inp, steps)
    ref = reference(shape, inp)
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cs.float().cpu().numpy(), ref["conv_out"])


@pytest.mark.parametrize("pro,epi", FUSIONS)
@pytest.mark.parametrize("shape,dtype,B,T", [(gi.TINY, "f32", 2, 5), (SMALL128, "bf16", 4, 4),
                                             (SMALL128, "bf16", 2, 16)])   # the widest block: 64 KB+ of LDS
def test_verify_fused(shape, dtype, B, T, pro, epi):
    _say(f"verify_ex {shape} {dtype} B={B} T={T} prologue={pro} epilogue={epi}")
    inp = fused_inputs(shape, B, T, 52, dtype, pro, epi)
    o, snap = run_verify(shape, dtype, inp, T)
    ref = reference(shape, inp)
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(snap[:, -1], ref["S"]) <= TOL[dtype]
    # the fused verify block equals the same tokens decoded one by one, bit for bit
    o_d, S_d, _ = run_decode(shape, dtype, inp, T)
    assert torch.equal(o, o_d)
    assert torch.equal(snap[:, -1], S_d)


@pytest.mark.parametrize("pro,epi", FUSIONS)
@pytest.mark.parametrize("shape,dtype,B,L", [(SMALL128, "bf16", 1, 200), (SMALL128, "f32", 2, 129),
                                             (gi.TINY_GQA, "bf16", 2, 70), (gi.TINY, "f32", 1, 64),
                                             (SMALL128, "bf16", 1, 1300),    # 1300: the 5-segment carry
                                             (SMALL128, "bf16", 2, 777)])    # two rows, segmented, ragged tail chunk
def test_prefill_fused(shape, dtype, B, L, pro, epi):
    _say(f"prefill_ex {shape} {dtype} B={B} L={L} prologue={pro} epilogue={epi}")
    inp = fused_inputs(shape, B, L, 53, dtype, pro, epi)
    o, S, cout = run_prefill(shape, dtype, inp)
    ref = reference(shape, inp)
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def test_prefill_fused_ragged_leaves_outside_tokens():
    """Packed sequences that stop short of L: the epilogue normalises only the
    tokens inside a sequence and leaves the tail of o as the caller left it."""
    shape, dtype = SMALL128, "bf16"
    lens = [70, 0, 130, 1, 64]
    cu = gi.cu_seqlens(lens)
    L = int(cu[-1]) + 37
    inp = fused_inputs(shape, 1, L, 54, dtype, True, True, N=len(lens))
    o, S, cout = run_prefill(shape, dtype, inp, cu=cu, o_fill=7.0)
    n_in = int(cu[-1])
    # the oracle packs sequences end to end over exactly cu[-1] tokens
    cut = dict(inp, qkv=inp["qkv"][:, :, :n_in], a=inp["a"][:, :n_in], b=inp["b"][:, :n_in],
               z=inp["z"][:, :n_in])
    ref = reference(shape, cut, cu=cu)
    assert rel_err(o[:, :n_in], ref["o"]) <= TOL[dtype]
    assert bool(torch.all(o[:, n_in:] == 7.0))
    assert rel_err(S, ref["S"]) <= TOL[dtype]
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def test_null_fusion_is_the_plain_call_bitexact():
    """fusion=NULL and a gdn_fusion with every field NULL both reproduce the
    plain entry points bit for bit."""
    shape, dtype, B, L = SMALL128, "bf16", 2, 150
    inp = fused_inputs(shape, B, L, 55, dtype, False, False)
    p = params(shape, dtype)
    args = [dev(inp[k], dtype) for k in ("qkv", "gate", "beta", "w", "conv0")]
    outs = []
    for mode in ("plain", "none", "empty"):
        S = dev(inp["S0"])
        o = torch.zeros((B, L, shape.Hv, shape.dv), device="cuda")
        cout = torch.zeros_like(args[4])
        ws = gdn.prefill_workspace(p, B, L, B)
        if mode == "plain":
            gdn.gdn_prefill(p, *args, cout, S, o, ws)
        else:
            gdn.gdn_prefill_ex(p, None if mode == "none" else gdn.GdnFusion(), *args, cout, S, o, ws)
        # one decode step on top of the prefill state
        od = torch.empty((B, 1, shape.Hv, shape.dv), device="cuda")
        cn = torch.empty_like(cout)
        q1 = dev(gi.qkv(shape, B, 1, 56, dtype), dtype)
        g1, b1 = dev(inp["gate"][:, :1], dtype), dev(inp["beta"][:, :1], dtype)
        if mode == "plain":
            gdn.gdn_decode_step(p, q1, g1, b1, args[3], cout, cn, S, od)
        else:
            gdn.gdn_decode_step_ex(p, None if mode == "none" else gdn.GdnFusion(), q1, g1, b1,
                                   args[3], cout, cn, S, od)
        torch.cuda.synchronize()
        outs.append((o, S, od, cn))
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)


@pytest.mark.parametrize("path", ["decode", "verify", "prefill"])
def test_fusions_at_saturating_inputs(path):
    """Raw gate/beta projections and gates z twenty times the usual spread (|x| up to about
    80): softplus and the sigmoids saturate, beta is nearly 0 or 1, some tokens' decay
    wipes the state and silu(z) is nearly z or 0. The prologue and epilogue must follow the
    oracle there too (MFMA prefill at 1300 tokens: the segmented carry)."""
    shape, dtype = SMALL128, "bf16"
    B, L = {"decode": (3, 10), "verify": (4, 8), "prefill": (1, 1300)}[path]
    _say(f"fusions at saturating inputs: {path}")
    inp = fused_inputs(shape, B, L, 56, dtype, True, True)
    for k in ("a", "b", "z"):
        inp[k] = gi.round_to(20.0 * inp[k].astype(np.float64), dtype)
    ref = reference(shape, inp)
    if path == "decode":
        o, S, _ = run_decode(shape, dtype, inp, L)
    elif path == "verify":
        o, snap = run_verify(shape, dtype, inp, L)
        S = snap[:, -1]
    else:
        o, S, _ = run_prefill(shape, dtype, inp)
    assert not torch.isnan(o).any()
    assert rel_err(o, ref["o"]) <= TOL[dtype]
    assert rel_err(S, ref["S"]) <= TOL[dtype]
