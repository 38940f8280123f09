"""CPU model of the chunked prefill's operand precision, the evidence behind the MFMA
operand type of the prefill kernels.

The chunked form of the gated delta rule (an exact rewrite of step 5 of "MNN Model
Support: Qwen3.5", §1.2, over chunks of 64 tokens) is evaluated in float64, except that
every operand of a dense product is rounded to the candidate MFMA input type first, with a
power-of-two scale that puts the operand's largest magnitude in [2^14, 2^15) (as the
kernels do for S, V, U and the deltas; exact to apply and undo). The fp32 parts of the
kernels (the triangular solve, the state, every accumulation) are modelled by rounding
their results to float32. The results are compared with the fp64 oracle's token-by-token
recurrence, with the error measure and budget of the GPU tests: max|err| / max|ref| <= 2e-3
for bf16 inputs.

bf16 operands (8 significant bits) miss the budget on these workloads; fp16 operands
(11 bits) meet it with room to spare. The GPU prefill therefore runs its products on
v_mfma_f32_16x16x32_f16.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import gdn_inputs as gi
import oracle

BUDGET = 2e-3


def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _fp16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def _bf16(x):
    return gi.round_bf16(x).astype(np.float64)


def _scaled(rnd):
    """Round x to a narrow type after scaling its largest magnitude into [2^14, 2^15)."""
    def f(x):
        x = np.asarray(x, np.float64)
        m = float(np.max(np.abs(x))) if x.size else 0.0
        if m == 0.0:
            return x.copy()
        e = math.frexp(m)[1] - 15
        return rnd(x * 2.0 ** -e) * 2.0 ** e
    return f


def _exp_for(x, top):
    """Exponent e with max|x 2^-e| in [2^(top - 1), 2^top) (0 for an all-zero x)."""
    m = float(np.max(np.abs(x))) if np.size(x) else 0.0
    return math.frexp(m)[1] - top if m > 0.0 else 0


def chunked_rounded(q, k, v, g, b, S0, rnd, C=64, state_top=None):
    """o [L, dv] and the final state of one V head, chunk by chunk, every product operand
    passed through rnd (q, k unit-norm and T, P, W bounded: the scale is a no-op for them).

    With state_top set (and rnd the plain narrow rounding), the state and Delta operands
    are rounded at the scale that puts their largest magnitude in [2^(state_top - 1),
    2^state_top) instead, both Delta operands (Delta and its decay-weighted copy) at
    Delta's scale: the carry kernel keeps these scales anywhere in a window of fp16's
    range rather than at its top."""
    if state_top is None:
        rs = rd = rnd
    else:
        def rs(x):
            e = _exp_for(x, state_top)
            return rnd(x * 2.0 ** -e) * 2.0 ** e

    L = q.shape[0]
    S = S0.copy()
    O = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        Q, K, V, G, Bt = q[sl], k[sl], v[sl], g[sl], b[sl]
        n = Q.shape[0]
        gam = _f32(np.cumsum(G))
        diff = gam[:, None] - gam[None, :]
        strict = np.tril(np.ones((n, n)), -1) > 0
        incl = np.tril(np.ones((n, n))) > 0
        Qr, Kr = rnd(Q), rnd(K)
        A = Bt[:, None] * np.exp(np.where(strict, diff, 0.0)) * (Kr @ Kr.T) * strict
        T = _f32(np.linalg.inv(np.eye(n) + A))
        W = _f32(rnd(T) @ rnd(np.exp(gam)[:, None] * Bt[:, None] * K))
        U = _f32(rnd(T) @ rnd(Bt[:, None] * V))
        P = np.exp(np.where(incl, diff, -np.inf)) * (Qr @ Kr.T)
        Sr = rs(S)
        Delta = _f32(rnd(U) - rnd(W) @ Sr)
        wD = np.exp(gam[-1] - gam)[:, None] * Delta
        if state_top is None:
            Dr, wDr = rnd(Delta), rnd(wD)
        else:
            e = _exp_for(Delta, state_top)
            Dr, wDr = rnd(Delta * 2.0 ** -e) * 2.0 ** e, rnd(wD * 2.0 ** -e) * 2.0 ** e
        O[sl] = _f32(np.exp(gam)[:, None] * (Qr @ Sr) + rnd(P) @ Dr)
        S = _f32(math.exp(gam[-1]) * S + Kr.T @ wDr)
    return O, S


def _case(seed, L, gate_scale=1.0, beta_high=False):
    sh = gi.Shape(Hk=1, Hv=2, dk=128, dv=128)
    x = gi.qkv(sh, 1, L, seed, "bf16")
    w = gi.conv_weight(sh, seed, "bf16")
    g = gi.round_to(gate_scale * gi.gate(sh, 1, L, seed, "bf16").astype(np.float64), "bf16")
    b = gi.beta(sh, 1, L, seed, "bf16")
    if beta_high:
        b = gi.round_to(0.5 + 0.5 * b.astype(np.float64), "bf16")
    zc, zs = np.zeros((1, sh.D, 3)), np.zeros((1, sh.Hv, 128, 128))
    op = oracle.OracleParams.of(sh)
    q, k, v = oracle.front_end(op, x, w, zc)
    ref = oracle.gdn_forward(op, x, g, b, w, zc, zs)
    h = 1   # V head 1 (K head 0)
    return (q[0, :, 0], k[0, :, 0], v[0, :, h], g[0, :, h].astype(np.float64),
            b[0, :, h].astype(np.float64), zs[0, h], ref["o"][0, :, h], ref["S"][0, h])


CASES = {
    "prefill_distributions_L512": lambda: _case(1002, 512),
    "long_memory_L512": lambda: _case(7, 512, gate_scale=0.01, beta_high=True),
}


def _err(a, r):
    return float(np.max(np.abs(a - r)) / np.max(np.abs(r)))


@pytest.fixture(scope="module")
def cases(oracle_lib):
    return {name: make() for name, make in CASES.items()}


def test_model_without_rounding_is_the_recurrence(cases):
    """With no rounding beyond fp32 the model reproduces the oracle (the algebra is exact)."""
    for name, (q, k, v, g, b, S0, o_ref, S_ref) in cases.items():
        O, S = chunked_rounded(q, k, v, g, b, S0, _f32)
        assert _err(O, o_ref) < 2e-5 and _err(S, S_ref) < 2e-5, name


def test_fp16_operands_meet_the_budget(cases):
    for name, (q, k, v, g, b, S0, o_ref, S_ref) in cases.items():
        O, S = chunked_rounded(q, k, v, g, b, S0, _scaled(_fp16))
        eo, es = _err(O, o_ref), _err(S, S_ref)
        assert eo <= BUDGET / 2 and es <= BUDGET / 2, (name, eo, es)


def test_bf16_operands_miss_the_budget(cases):
    worst = 0.0
    for name, (q, k, v, g, b, S0, o_ref, S_ref) in cases.items():
        O, S = chunked_rounded(q, k, v, g, b, S0, _scaled(_bf16))
        worst = max(worst, _err(O, o_ref), _err(S, S_ref))
    assert worst > BUDGET, worst


def test_fp16_operands_anywhere_in_the_carried_window(cases):
    """The carry keeps the state's and Delta's power-of-two scales from chunk to chunk while
    their largest magnitude stays in [2^6, 2^15): with it at the bottom of that window the
    fp16 operands give the same error as with it at the top (fp16's relative precision
    does not depend on the scale until values fall below its smallest normal, 2^-14)."""
    for name, (q, k, v, g, b, S0, o_ref, S_ref) in cases.items():
        Ot, St = chunked_rounded(q, k, v, g, b, S0, _fp16, state_top=15)
        Ol, Sl = chunked_rounded(q, k, v, g, b, S0, _fp16, state_top=7)
        et, el = (_err(Ot, o_ref), _err(St, S_ref)), (_err(Ol, o_ref), _err(Sl, S_ref))
        assert max(el) <= BUDGET / 2, (name, el)
        for x, y in zip(el, et):
            assert abs(x - y) <= 0.01 * y, (name, el, et)
