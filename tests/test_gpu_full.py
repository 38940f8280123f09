"""GPU parity at the full workload sizes, in the launch configuration bench.py
times. The HIP path runs the whole workload; the fp64 oracle computes a sample
of (sequence, V head) units (both V heads of a GQA pair, first/last heads and
sequences) and every raw conv-state value, which are compared exactly."""
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


def _mask(N, Hv, units):
    m = np.zeros((N, Hv), bool)
    for n, h in units:
        m[n, h] = True
    return m


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
    units = [(0, 0), (0, 1), (17, 14), (17, 15), (63, 30), (63, 31), (40, 7)]
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, c0, S0, unit_mask=_mask(B, SH.Hv, units))
    bi = [u[0] for u in units]
    hi = [u[1] for u in units]
    assert rel_err(o[bi, :, hi], ref["o"][bi, :, hi]) <= TOL["bf16"]
    assert rel_err(S[bi, hi], ref["S"][bi, hi]) <= TOL["bf16"]
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
    heads = [0, 1, 16, 17, 31]
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, np.zeros((1, SH.D, 3)), np.zeros((1, SH.Hv, 128, 128)),
                             unit_mask=_mask(1, SH.Hv, [(0, h) for h in heads]))
    assert not torch.isnan(o).any()
    assert rel_err(o[0][:, heads], ref["o"][0][:, heads]) <= TOL["bf16"]
    assert rel_err(S[0, heads], ref["S"][0, heads]) <= TOL["bf16"]
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
    units = [(0, 0), (0, 31), (3, 8), (3, 9), (7, 0), (int(np.argmax(lens)), 20)]
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, np.zeros((N, SH.D, 3)), np.zeros((N, SH.Hv, 128, 128)),
                             cu_seqlens=cu, unit_mask=_mask(N, SH.Hv, units))
    assert not torch.isnan(o).any()
    for n, h in units:
        s, e = int(cu[n]), int(cu[n + 1])
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
    units = [(0, 0), (0, 1), (64, 16), (64, 17), (127, 31), (99, 5)]
    ref = oracle.gdn_forward(oparams(SH), x, g, b, w, c0, S0, snapshots=True,
                             unit_mask=_mask(B, SH.Hv, units))
    bi = [u[0] for u in units]
    hi = [u[1] for u in units]
    assert rel_err(o[bi, :, hi], ref["o"][bi, :, hi]) <= TOL["bf16"]
    assert rel_err(snap[bi, :, hi], ref["snap"][bi, :, hi]) <= TOL["bf16"]
    S_ref, c_ref = oracle.verify_commit(oparams(SH), acc, x, c0, ref["snap"])
    assert rel_err(S_out[bi, hi], S_ref[bi, hi]) <= TOL["bf16"]
    assert np.array_equal(c_out.float().cpu().numpy(), c_ref)
    # every row's committed state is exactly its selected snapshot
    sel = snap[torch.arange(B, device="cuda"), torch.from_numpy(acc).long().cuda()]
    assert torch.equal(S_out, sel)
