"""GPU parity at the full workload sizes, in the launch configuration bench.py
times. The HIP path runs the whole workload and the fp64 oracle computes every
(sequence, V head) unit of it (about 10 GFLOP/s on 16 host threads: decode's 69
GFLOP, the ragged prompt's 119 GFLOP and the 4096-token prompt's 17 GFLOP each
take seconds), so every output, every final state or snapshot, and every raw
conv-state value (compared exactly) is checked, whichever workgroup produced it."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_sequence_amd as gdn
import oracle
from gpu_cases import TOL, dev, oparams, params, rel_err

pytestmark = pytest.mark.gpu
SH = gi.QWEN


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()
    oracle.build_oracle(force=False)


def test_decode_B64_256_steps():
    seed, B, steps = gi.WORKLOADS[1].seed, gi.DECODE_B, gi.DECODE_STEPS
    print(f"decode full B={B} steps={steps}", flush=True)
    p = params(SH, "bf16")
    x = np.concatenate([gi.qkv(SH, B, 1, seed, "bf16", step=s) for s in range(steps)], axis=2)
    g = np.concatenate([gi.gate(SH, B, 1, seed, "bf16", step=s) for s in range(steps)], axis=1)
    b = np.concatenate([gi.beta(SH, B, 1, seed, "bf16", step=s) for s in range(steps)], axis=1)
    w = gi.conv_weight(SH, seed, "bf16")
    S0 = gi.state0(SH, B, seed, 0.1)
    c0 = gi.conv_state0(SH, B, seed, 1.0, "bf16")
    S = dev(S0)
    cs = dev(c0, "bf16")
    wd = dev(w, "bf16")
    xd, gd, bd = dev(x, "bf16"), dev(g, "bf16"), dev(b, "bf16")
    o = torch.empty((B, steps, SH.Hv, SH.dv), device="cuda")
    for t in range(steps):
        cn = torch.empty_like(cs)
        ot = torch.empty((B, 1, SH.Hv, SH.dv), device="cuda")
        gdn.gdn_decode_step(p, xd[:, :, t:t + 1].contiguous(), gd[:, t:t + 1].contiguous(),
                            bd[:, t:t + 1].contiguous(), wd, cs, cn, S, ot)
        o[:, t:t + 1] = ot
        cs = cn
    torch.cuda.synchronize()
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, c0, S0)
    assert rel_err(o, ref["o"]) <= TOL["bf16"]
    assert rel_err(S, ref["S"]) <= TOL["bf16"]
    for bb in (0, B - 1):   # per-sequence errors stay within the bound too (not only the global max)
        assert rel_err(o[bb], ref["o"][bb]) <= TOL["bf16"], bb
    assert np.array_equal(cs.float().cpu().numpy(), ref["conv_out"])


def _prefill(x, g, b, w, N, cu=None):
    p = params(SH, "bf16")
    L = x.shape[2]
    S = torch.zeros((N, SH.Hv, SH.dk, SH.dv), device="cuda")
    o = torch.full((1, L, SH.Hv, SH.dv), float("nan"), device="cuda")
    c0 = torch.zeros((N, SH.D, SH.K - 1), device="cuda", dtype=torch.bfloat16)
    cout = torch.empty_like(c0)
    ws = gdn.prefill_workspace(p, 1, L, N)
    gdn.gdn_prefill(p, dev(x, "bf16"), dev(g, "bf16"), dev(b, "bf16"), dev(w, "bf16"), c0, cout, S, o,
                    ws, cu_seqlens=None if cu is None else dev(cu))
    torch.cuda.synchronize()
    return o, S, cout


def test_prefill_L4096():
    seed, L = gi.WORKLOADS[2].seed, gi.PREFILL_L
    print(f"prefill full L={L}", flush=True)
    x = gi.qkv(SH, 1, L, seed, "bf16")
    g = gi.gate(SH, 1, L, seed, "bf16")
    b = gi.beta(SH, 1, L, seed, "bf16")
    w = gi.conv_weight(SH, seed, "bf16")
    o, S, cout = _prefill(x, g, b, w, 1)
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, np.zeros((1, SH.D, 3)), np.zeros((1, SH.Hv, 128, 128)))
    assert not torch.isnan(o).any()
    assert rel_err(o, ref["o"]) <= TOL["bf16"]
    assert rel_err(S, ref["S"]) <= TOL["bf16"]
    for h in range(SH.Hv):   # every head, i.e. every (slice, slot) of both carry passes
        assert rel_err(o[0, :, h], ref["o"][0, :, h]) <= TOL["bf16"], h
        assert rel_err(S[0, h], ref["S"][0, h]) <= TOL["bf16"], h
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def test_prefill_L16384():
    """Four times the 4096-token prompt: the segmented carry with about 50 chunks per
    segment and the workspace at that size; every head against the oracle."""
    seed, L = gi.WORKLOADS[2].seed + 1, 4 * gi.PREFILL_L
    print(f"prefill full L={L}", flush=True)
    x = gi.qkv(SH, 1, L, seed, "bf16")
    g = gi.gate(SH, 1, L, seed, "bf16")
    b = gi.beta(SH, 1, L, seed, "bf16")
    w = gi.conv_weight(SH, seed, "bf16")
    o, S, cout = _prefill(x, g, b, w, 1)
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, np.zeros((1, SH.D, 3)), np.zeros((1, SH.Hv, 128, 128)))
    assert not torch.isnan(o).any()
    for h in range(SH.Hv):
        assert rel_err(o[0, :, h], ref["o"][0, :, h]) <= TOL["bf16"], h
        assert rel_err(S[0, h], ref["S"][0, h]) <= TOL["bf16"], h
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def test_ragged_prefill_8_sequences():
    seed = gi.WORKLOADS[3].seed
    lens = gi.seq_lens(gi.RAGGED_N, gi.RAGGED_LO, gi.RAGGED_HI, seed)
    cu = gi.cu_seqlens(lens)
    L, N = int(cu[-1]), gi.RAGGED_N
    print(f"ragged prefill full lens={lens.tolist()} total={L}", flush=True)
    x = gi.qkv(SH, 1, L, seed, "bf16")
    g = gi.gate(SH, 1, L, seed, "bf16")
    b = gi.beta(SH, 1, L, seed, "bf16")
    w = gi.conv_weight(SH, seed, "bf16")
    o, S, cout = _prefill(x, g, b, w, N, cu=cu)
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, np.zeros((N, SH.D, 3)), np.zeros((N, SH.Hv, 128, 128)),
                             cu_seqlens=cu)
    assert not torch.isnan(o).any()
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(SH.Hv):
            assert rel_err(o[0, s:e, h], ref["o"][0, s:e, h]) <= TOL["bf16"], (n, h)
            assert rel_err(S[n, h], ref["S"][n, h]) <= TOL["bf16"], (n, h)
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def _fused_prefill_case(seed, L, N, cu=None):
    """The fused workloads' inputs (raw a/b through the gate/beta prologue, gated RMSNorm
    with z): device results and the oracle's."""
    x = gi.qkv(SH, 1, L, seed, "bf16")
    a_raw, b_raw = gi.a_raw(SH, 1, L, seed, "bf16"), gi.b_raw(SH, 1, L, seed, "bf16")
    A_log, dt_bias = gi.a_log(SH, seed, "bf16"), gi.dt_bias(SH, seed, "bf16")
    z, nw = gi.z_gate(SH, 1, L, seed, "bf16"), gi.norm_weight(SH, seed, "bf16")
    w = gi.conv_weight(SH, seed, "bf16")
    p = params(SH, "bf16")
    S = torch.zeros((N, SH.Hv, SH.dk, SH.dv), device="cuda")
    o = torch.full((1, L, SH.Hv, SH.dv), float("nan"), device="cuda")
    c0 = torch.zeros((N, SH.D, SH.K - 1), device="cuda", dtype=torch.bfloat16)
    cout = torch.empty_like(c0)
    ws = gdn.prefill_workspace(p, 1, L, N)
    fus = gdn.GdnFusion(dev(A_log, "bf16"), dev(dt_bias, "bf16"), dev(z, "bf16"), dev(nw, "bf16"), 1e-6)
    gdn.gdn_prefill_ex(p, fus, dev(x, "bf16"), dev(a_raw, "bf16"), dev(b_raw, "bf16"), dev(w, "bf16"), c0, cout,
                       S, o, ws, cu_seqlens=None if cu is None else dev(cu))
    torch.cuda.synchronize()
    g, b = oracle.gate_beta(a_raw, b_raw, A_log, dt_bias)
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, np.zeros((N, SH.D, 3)), np.zeros((N, SH.Hv, 128, 128)),
                             cu_seqlens=cu)
    ref["o"] = oracle.gated_rmsnorm(ref["o"], z, nw, 1e-6)
    return o, S, cout, ref


def test_prefill_L4096_fused():
    """The gated RMSNorm in the carry's output store (whole-head workgroups in both
    passes of the segmented carry), every head of the 4096-token prompt."""
    seed, L = gi.WORKLOADS[2].seed, gi.PREFILL_L
    print(f"prefill fused full L={L}", flush=True)
    o, S, cout, ref = _fused_prefill_case(seed, L, 1)
    assert not torch.isnan(o).any()
    for h in range(SH.Hv):
        assert rel_err(o[0, :, h], ref["o"][0, :, h]) <= TOL["bf16"], h
        assert rel_err(S[0, h], ref["S"][0, h]) <= TOL["bf16"], h
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def test_ragged_prefill_fused():
    seed = gi.WORKLOADS[3].seed
    lens = gi.seq_lens(gi.RAGGED_N, gi.RAGGED_LO, gi.RAGGED_HI, seed)
    cu = gi.cu_seqlens(lens)
    L, N = int(cu[-1]), gi.RAGGED_N
    print(f"ragged prefill fused full total={L}", flush=True)
    o, S, cout, ref = _fused_prefill_case(seed, L, N, cu=cu)
    assert not torch.isnan(o).any()
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(SH.Hv):
            assert rel_err(o[0, s:e, h], ref["o"][0, s:e, h]) <= TOL["bf16"], (n, h)
            assert rel_err(S[n, h], ref["S"][n, h]) <= TOL["bf16"], (n, h)
    assert np.array_equal(cout.float().cpu().numpy(), ref["conv_out"])


def test_verify_B128_T4_and_commit():
    seed, B, T = gi.WORKLOADS[4].seed, gi.VERIFY_B, gi.VERIFY_T
    print(f"verify full B={B} T={T}", flush=True)
    p = params(SH, "bf16")
    x = gi.qkv(SH, B, T, seed, "bf16")
    g = gi.gate(SH, B, T, seed, "bf16")
    b = gi.beta(SH, B, T, seed, "bf16")
    w = gi.conv_weight(SH, seed, "bf16")
    S0 = gi.state0(SH, B, seed, 0.1)
    c0 = gi.conv_state0(SH, B, seed, 1.0, "bf16")
    acc = gi.accept_len(B, T, seed)
    snap = torch.empty((B, T, SH.Hv, SH.dk, SH.dv), device="cuda")
    o = torch.empty((B, T, SH.Hv, SH.dv), device="cuda")
    S_in = dev(S0)
    cin = dev(c0, "bf16")
    xd = dev(x, "bf16")
    gdn.gdn_verify_block(p, xd, dev(g, "bf16"), dev(b, "bf16"), dev(w, "bf16"), cin, S_in, snap, o)
    S_out = torch.empty_like(S_in)
    c_out = torch.empty_like(cin)
    gdn.gdn_verify_commit(p, dev(acc), xd, cin, snap, c_out, S_out)
    torch.cuda.synchronize()
    assert torch.equal(S_in, dev(S0))   # S_in is read only
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, c0, S0, snapshots=True)
    assert rel_err(o, ref["o"]) <= TOL["bf16"]
    assert rel_err(snap, ref["snap"]) <= TOL["bf16"]
    S_ref, c_ref = oracle.verify_commit(oparams(SH), acc, x, c0, ref["snap"])
    assert rel_err(S_out, S_ref) <= TOL["bf16"]
    assert np.array_equal(c_out.float().cpu().numpy(), c_ref)
    # every row's committed state is exactly its selected snapshot
    sel = snap[torch.arange(B, device="cuda"), torch.from_numpy(acc).long().cuda()]
    assert torch.equal(S_out, sel)
