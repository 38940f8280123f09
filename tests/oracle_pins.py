"""Pins of the fp64 oracle against things other than itself.

Each pin is a plain function that raises AssertionError on failure, so that
test_oracle_pins.py can run them one by one and test_oracle_mutations.py can
show that every planted mistake makes at least one of them fail.

What pins what (passages of "MNN Model Support: Qwen3.5"):
  * §1.2 Step 5 (the recurrence):
      - a two-token example worked by hand (tests/golden/hand_worked_two_tokens.json);
      - exact-rational brute force in fractions.Fraction using the
        generalised-Householder form  S_t = a_t (I - b_t k k^T) S_{t-1} + b_t k v^T;
      - the Kronecker (dense linear map) form  vec(S_t) = (a(I - b k k^T) (x) I) vec(S_{t-1}) + b vec(k v^T);
      - the chunked WY/UT form (an exact algebraic rewrite, different algorithm) at C = 4, 16, 64;
      - closed forms: o = b (k.q) v from a zero state; b = 0 & g = 0 keeps S; b = 1 with a
        unit key recalls v exactly after the write; b = 0 is pure decay exp(Gamma_t) S_0;
      - the Widrow-Hoff LMS special case (a = 1) and the spectral-norm bound.
  * §1.2 Step 1 (conv + SiLU): scipy/numpy correlation and scipy.special.expit, one-hot taps,
    split/carry of the conv state.
  * §1.2 Steps 2-4 and §1.3 (split, repeat_interleave GQA, L2 norm, 1/sqrt(dk)): index
    probes against numpy.repeat (numpy's repeat_interleave), norms, and an end-to-end probe
    whose output identifies which K head each V head read.
  * whole layer: composition of the pinned pieces; carry invariants (split calls, ragged
    packing, snapshots, commit).
  * §1.2 gate/beta parameterisation: torch softplus/sigmoid in fp64, closed forms
    (softplus(0) = ln 2, sigmoid(0) = 1/2, sigmoid(b) + sigmoid(-b) = 1), gate <= 0.
  * §2 gated RMSNorm: torch rms_norm and silu in fp64, scale invariance, zero gate.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import scipy.special
import scipy.signal

import gdn_inputs as gi
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def _frac(x):
    return Fraction(x)


# ---------------------------------------------------------------------------
# Step 5: the recurrence core
# ---------------------------------------------------------------------------
def pin_hand_worked():
    with open(os.path.join(GOLDEN, "hand_worked_two_tokens.json")) as f:
        gd = json.load(f)
    alpha = [float(_frac(a)) for a in gd["alpha"]]
    g = np.log(alpha)
    beta = [float(_frac(b)) for b in gd["beta"]]
    k = np.array([[float(_frac(x)) for x in r] for r in gd["k"]])
    q = np.array([[float(_frac(x)) for x in r] for r in gd["q"]])
    v = np.array([[float(_frac(x)) for x in r] for r in gd["v"]])
    o_ref = np.array([[float(_frac(x)) for x in r] for r in gd["o"]])
    S_ref = np.array([[float(_frac(x)) for x in r] for r in gd["S_final"]])
    o, S = oracle.delta_rule(q, k, v, g, beta, np.zeros((2, 2)))
    assert _rel(o, o_ref) < 1e-14, (o, o_ref)
    assert _rel(S, S_ref) < 1e-14, (S, S_ref)


def _householder_exact(ks, qs, vs, alphas, betas, S0):
    """Exact rational evaluation of S_t = a(I - b k k^T) S_{t-1} + b k v^T, o_t = S_t^T q_t."""
    dk = len(S0)
    dv = len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for k, q, v, a, b in zip(ks, qs, vs, alphas, betas):
        # M = a (I - b k k^T)
        M = [[a * ((1 if i == j else 0) - b * k[i] * k[j]) for j in range(dk)] for i in range(dk)]
        S = [[sum(M[i][m] * S[m][j] for m in range(dk)) + b * k[i] * v[j] for j in range(dv)]
             for i in range(dk)]
        outs.append([sum(S[i][j] * q[i] for i in range(dk)) for j in range(dv)])
    return outs, S


def pin_rational_brute_force():
    with open(os.path.join(GOLDEN, "rational_cases.json")) as f:
        rc = json.load(f)
    units = [[_frac(x) for x in u] for u in rc["unit_vectors"]]
    for u in units:
        assert sum(x * x for x in u) == 1
    alphas = [_frac(a) for a in rc["alphas"]]
    betas = [_frac(b) for b in rc["betas"]]
    values = [[_frac(x) for x in r] for r in rc["values"]]
    S0 = [[_frac(x) for x in r] for r in rc["S0"]]
    half = Fraction(1, 2)  # 1/sqrt(dk) with dk = 4
    L = 12
    ks = [units[(3 * t + 1) % len(units)] for t in range(L)]
    qs = [[half * x for x in units[(5 * t + 2) % len(units)]] for t in range(L)]
    vs = [values[t % len(values)] for t in range(L)]
    al = [alphas[(t + 1) % len(alphas)] for t in range(L)]
    be = [betas[(2 * t) % len(betas)] for t in range(L)]
    o_ex, S_ex = _householder_exact(ks, qs, vs, al, be, S0)
    o, S = oracle.delta_rule(np.array(qs, float), np.array(ks, float), np.array(vs, float),
                             np.log(np.array(al, float)), np.array(be, float), np.array(S0, float))
    assert _rel(o, np.array(o_ex, float)) < 1e-13
    assert _rel(S, np.array(S_ex, float)) < 1e-13


def _rand_core(rng, L, dk, dv, g_scale=1.0, s0_std=0.5):
    q = rng.standard_normal((L, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True) * math.sqrt(dk)
    k = rng.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, dv))
    g = -g_scale * np.logaddexp(0, rng.standard_normal(L))
    b = scipy.special.expit(rng.standard_normal(L))
    S0 = s0_std * rng.standard_normal((dk, dv))
    return q, k, v, g, b, S0


def pin_kronecker_form():
    rng = np.random.default_rng(11)
    for L, dk, dv in ((24, 8, 6), (16, 6, 6)):
        q, k, v, g, b, S0 = _rand_core(rng, L, dk, dv)
        s = S0.reshape(-1).copy()  # row-major vec: index i*dv + j
        outs = []
        for t in range(L):
            a = math.exp(g[t])
            A = a * (np.eye(dk) - b[t] * np.outer(k[t], k[t]))
            s = np.kron(A, np.eye(dv)) @ s + b[t] * np.outer(k[t], v[t]).reshape(-1)
            outs.append(np.kron(q[t][None, :], np.eye(dv)) @ s)
        o, S = oracle.delta_rule(q, k, v, g, b, S0)
        assert _rel(o, np.array(outs)) < 1e-12
        assert _rel(S, s.reshape(dk, dv)) < 1e-12


def chunked_form(q, k, v, g, b, S0, C):
    """The chunked (WY / UT transform) rewrite of the recurrence, fp64 numpy.

    Inside a chunk with cumulative log-decay Gam_t = sum_{s<=t} g_s:
      A_ts = b_t exp(Gam_t - Gam_s) (k_t . k_s) for s < t,   T = (I + A)^-1
      W = T diag(b exp(Gam)) K,  U = T diag(b) V,  Delta = U - W S0
      O = diag(exp(Gam)) Q S0 + (M o Q K^T) Delta,  M_ts = exp(Gam_t - Gam_s) (s <= t)
      S_C = exp(Gam_C) S0 + K^T diag(exp(Gam_C - Gam)) Delta
    """
    L = q.shape[0]
    S = S0.copy()
    O = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        Q, K, V, G, B = q[sl], k[sl], v[sl], g[sl], b[sl]
        n = Q.shape[0]
        Gam = np.cumsum(G)
        diff = Gam[:, None] - Gam[None, :]
        lower = np.tril(np.ones((n, n)), -1)
        A = B[:, None] * np.exp(np.where(lower > 0, diff, 0.0)) * (K @ K.T) * lower
        T = np.linalg.inv(np.eye(n) + A)
        W = T @ (np.diag(B * np.exp(Gam)) @ K)
        U = T @ (np.diag(B) @ V)
        Delta = U - W @ S
        M = np.exp(np.where(np.tril(np.ones((n, n))) > 0, diff, -np.inf))
        O[sl] = np.exp(Gam)[:, None] * (Q @ S) + (M * (Q @ K.T)) @ Delta
        S = math.exp(Gam[-1]) * S + K.T @ (np.exp(Gam[-1] - Gam)[:, None] * Delta)
    return O, S


def pin_chunked_form():
    rng = np.random.default_rng(12)
    for L, C in ((64, 4), (100, 16), (130, 64)):
        q, k, v, g, b, S0 = _rand_core(rng, L, 16, 12, g_scale=0.1)
        O, S = chunked_form(q, k, v, g, b, S0, C)
        o, So = oracle.delta_rule(q, k, v, g, b, S0)
        assert _rel(o, O) < 1e-11, (L, C, _rel(o, O))
        assert _rel(So, S) < 1e-11, (L, C, _rel(So, S))


def pin_closed_forms():
    rng = np.random.default_rng(13)
    dk, dv = 8, 5
    # (1) one step from the zero state: o = beta (k.q) v
    q, k, v, g, b, _ = _rand_core(rng, 1, dk, dv)
    o, _ = oracle.delta_rule(q, k, v, g, b, np.zeros((dk, dv)))
    assert _rel(o[0], b[0] * float(k[0] @ q[0]) * v[0]) < 1e-14
    # (2) beta = 0, g = 0: S unchanged bit for bit, o = S^T q
    q, k, v, _, _, S0 = _rand_core(rng, 6, dk, dv)
    o, S = oracle.delta_rule(q, k, v, np.zeros(6), np.zeros(6), S0)
    assert np.array_equal(S, S0)
    assert _rel(o, q @ S0) < 1e-14
    # (3) beta = 1 with unit keys: after the write S^T k = v, for any decay
    q, k, v, g, _, S0 = _rand_core(rng, 7, dk, dv)
    o, S, snap = oracle.delta_rule(q, k, v, g, np.ones(7), S0, snapshots=True)
    for t in range(7):
        assert _rel(snap[t].T @ k[t], v[t]) < 1e-13
    # (4) beta = 0: pure decay exp(Gamma_t) S0
    o, S, snap = oracle.delta_rule(q, k, v, g, np.zeros(7), S0, snapshots=True)
    Gam = np.cumsum(g)
    for t in range(7):
        assert _rel(snap[t], math.exp(Gam[t]) * S0) < 1e-14
        assert _rel(o[t], math.exp(Gam[t]) * (q[t] @ S0)) < 1e-13
    # (5) total forgetting (exp(g) underflows to exactly 0): every token starts from the
    # zero state whatever came before, so S_t = beta_t k_t v_t^T and o_t = beta_t (k_t.q_t) v_t
    q, k, v, _, b, S0 = _rand_core(rng, 5, dk, dv)
    o, S, snap = oracle.delta_rule(q, k, v, np.full(5, -1.0e4), b, S0, snapshots=True)
    for t in range(5):
        assert _rel(snap[t], b[t] * np.outer(k[t], v[t])) < 1e-14
        assert _rel(o[t], b[t] * float(k[t] @ q[t]) * v[t]) < 1e-13


def pin_lms_and_norm_bound():
    """alpha = 1 is the Widrow-Hoff LMS rule: weights W, input k, target v,
    error e = v - W^T k, update W += beta k e^T. And for beta in [0, 2] with unit
    keys the spectral norm obeys ||S_t|| <= alpha ||S_{t-1}|| + beta ||v_t||."""
    rng = np.random.default_rng(14)
    L, dk, dv = 20, 6, 4
    q, k, v, g, b, S0 = _rand_core(rng, L, dk, dv)
    W = S0.copy()
    outs = []
    for t in range(L):
        err = v[t] - W.T @ k[t]
        W = W + b[t] * np.outer(k[t], err)
        outs.append(W.T @ q[t])
    o, S = oracle.delta_rule(q, k, v, np.zeros(L), b, S0)
    assert _rel(o, np.array(outs)) < 1e-13 and _rel(S, W) < 1e-13
    b2 = 2.0 * scipy.special.expit(rng.standard_normal(L))
    o, S, snap = oracle.delta_rule(q, k, v, g, b2, S0, snapshots=True)
    prev = np.linalg.norm(S0, 2)
    for t in range(L):
        cur = np.linalg.norm(snap[t], 2)
        assert cur <= math.exp(g[t]) * prev + b2[t] * np.linalg.norm(v[t]) + 1e-12
        prev = cur


# ---------------------------------------------------------------------------
# Step 1: conv + SiLU
# ---------------------------------------------------------------------------
def _conv_case(rng, shape, B, L):
    x = rng.standard_normal((B, shape.D, L))
    w = 0.5 * rng.standard_normal((shape.D, 1, shape.K))
    st = rng.standard_normal((B, shape.D, shape.K - 1))
    return x, w, st


def pin_conv_library():
    """Pre-activation = numpy 'valid' cross-correlation of concat(state, x) with w;
    SiLU = x * scipy.special.expit(x). New state = last K-1 window entries."""
    rng = np.random.default_rng(21)
    shape = gi.Shape(Hk=1, Hv=2, dk=3, dv=2, K=4)
    p = oracle.OracleParams.of(shape)
    x, w, st = _conv_case(rng, shape, 2, 9)
    y, cout = oracle.conv1d_silu(p, x, w, st)
    for b in range(2):
        for c in range(shape.D):
            xh = np.concatenate([st[b, c], x[b, c]])
            pre = np.correlate(xh, w[c, 0], mode="valid")
            assert _rel(y[b, c], pre * scipy.special.expit(pre)) < 1e-14
            pre2 = scipy.signal.lfilter(w[c, 0][::-1], [1.0], xh)[shape.K - 1:]
            assert _rel(pre, pre2) < 1e-13
            assert np.array_equal(cout[b, c], xh[-(shape.K - 1):])


def pin_conv_onehot_and_carry():
    rng = np.random.default_rng(22)
    shape = gi.Shape(Hk=1, Hv=1, dk=2, dv=3, K=4)
    p = oracle.OracleParams.of(shape)
    x, w, st = _conv_case(rng, shape, 1, 7)
    w_cur = np.zeros_like(w); w_cur[:, 0, shape.K - 1] = 1.0   # identity
    y, _ = oracle.conv1d_silu(p, x, w_cur, st)
    assert _rel(y, x * scipy.special.expit(x)) < 1e-15
    w_old = np.zeros_like(w); w_old[:, 0, 0] = 1.0             # delay of K-1
    y, _ = oracle.conv1d_silu(p, x, w_old, st)
    xh = np.concatenate([st, x], axis=2)[:, :, :7]
    assert _rel(y, xh * scipy.special.expit(xh)) < 1e-15
    # split / carry: conv over 7 tokens == 3 tokens then 4 tokens with the state carried
    y_all, c_all = oracle.conv1d_silu(p, x, w, st)
    y1, c1 = oracle.conv1d_silu(p, x[:, :, :3], w, st)
    y2, c2 = oracle.conv1d_silu(p, x[:, :, 3:], w, c1)
    assert np.array_equal(np.concatenate([y1, y2], axis=2), y_all)
    assert np.array_equal(c2, c_all)
    # a 1-token call keeps the two newest state entries and appends the token
    _, c3 = oracle.conv1d_silu(p, x[:, :, :1], w, st)
    assert np.array_equal(c3[:, :, :-1], st[:, :, 1:]) and np.array_equal(c3[:, :, -1], x[:, :, 0])


# ---------------------------------------------------------------------------
# Steps 2-4 and reverse GQA
# ---------------------------------------------------------------------------
def pin_front_end_mapping_and_norms():
    rng = np.random.default_rng(31)
    shape = gi.TINY_GQA  # Hk = 2, Hv = 4, f = 2
    p = oracle.OracleParams.of(shape)
    B, L = 1, 5
    x, w, st = _conv_case(rng, shape, B, L)
    q, k, v = oracle.front_end(p, x, w, st)
    y, _ = oracle.conv1d_silu(p, x, w, st)
    Hk, Hv, dk, dv = shape.Hk, shape.Hv, shape.dk, shape.dv
    yq = y[0, :Hk * dk].reshape(Hk, dk, L).transpose(2, 0, 1)          # [L, Hk, dk]
    yk = y[0, Hk * dk:2 * Hk * dk].reshape(Hk, dk, L).transpose(2, 0, 1)
    yv = y[0, 2 * Hk * dk:].reshape(Hv, dv, L).transpose(2, 0, 1)       # [L, Hv, dv]
    f = Hv // Hk
    eq = np.repeat(yq, f, axis=1)   # numpy's repeat_interleave
    ek = np.repeat(yk, f, axis=1)
    # norms: ||k_hat|| = 1, ||q_hat|| = 1/sqrt(dk) (to eps)
    assert np.allclose(np.linalg.norm(k[0], axis=-1), 1.0, atol=1e-6)
    assert np.allclose(np.linalg.norm(q[0], axis=-1), 1.0 / math.sqrt(dk), atol=1e-6)
    # directions: q_hat, k_hat parallel to the conv output of K/Q head h // f
    cq = np.einsum("thi,thi->th", q[0], eq) / (np.linalg.norm(q[0], axis=-1) * np.linalg.norm(eq, axis=-1))
    ck = np.einsum("thi,thi->th", k[0], ek) / (np.linalg.norm(k[0], axis=-1) * np.linalg.norm(ek, axis=-1))
    assert np.all(cq > 1 - 1e-12) and np.all(ck > 1 - 1e-12)
    assert np.array_equal(v[0], yv)
    # with use_qk_l2norm off: q_hat = y_q / sqrt(dk) and k_hat = y_k exactly
    p_off = oracle.OracleParams.of(shape, use_qk_l2norm=False)
    q0, k0, _ = oracle.front_end(p_off, x, w, st)
    assert _rel(q0[0], eq / math.sqrt(dk)) < 1e-15 and np.array_equal(k0[0], ek)


def pin_gqa_end_to_end_probe():
    """One token from a zero state with an identity conv: o_h = beta_h (k_hat.q_hat) v_h where
    k_hat, q_hat come from K head h // f. Each K head gets a different angle between its key
    and query, so the output names the K head each V head read."""
    shape = gi.TINY_GQA
    p = oracle.OracleParams.of(shape)
    Hk, Hv, dk, dv, K = shape.Hk, shape.Hv, shape.dk, shape.dv, shape.K
    D = shape.D
    x = np.zeros((1, D, 1))
    a_q = 1.5
    angles = [(0.7, 0.3), (0.2, 1.1)]
    for j in range(Hk):
        x[0, j * dk + 0, 0] = a_q                       # q of K head j along e0
        x[0, Hk * dk + j * dk + 0, 0] = angles[j][0]     # k of K head j in the e0/e1 plane
        x[0, Hk * dk + j * dk + 1, 0] = angles[j][1]
    rng = np.random.default_rng(32)
    xv = rng.standard_normal((Hv, dv))
    x[0, 2 * Hk * dk:, 0] = xv.reshape(-1)
    w = np.zeros((D, 1, K)); w[:, 0, K - 1] = 1.0
    st = np.zeros((1, D, K - 1))
    gate = np.full((1, 1, Hv), -0.3)
    beta = np.array([0.9, 0.6, 0.3, 0.75]).reshape(1, 1, Hv)
    res = oracle.gdn_forward(p, x, gate, beta, w, st, np.zeros((1, Hv, dk, dv)))
    silu = lambda z: z * scipy.special.expit(z)
    s0 = silu(0.0)
    for h in range(Hv):
        j = h // (Hv // Hk)
        kv = np.full(dk, s0); kv[0] = silu(angles[j][0]); kv[1] = silu(angles[j][1])
        qv = np.full(dk, s0); qv[0] = silu(a_q)
        kh = kv / math.sqrt(kv @ kv + 1e-6)
        qh = qv / math.sqrt(qv @ qv + 1e-6) / math.sqrt(dk)
        expect = beta[0, 0, h] * (kh @ qh) * silu(xv[h])
        assert _rel(res["o"][0, 0, h], expect) < 1e-13, h


# ---------------------------------------------------------------------------
# Whole layer: composition and carry invariants
# ---------------------------------------------------------------------------
def _layer_case(shape, B, L, seed, s0_std=0.1, conv_std=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, shape.D, L))
    w = 0.5 * rng.standard_normal((shape.D, 1, shape.K))
    g = -np.logaddexp(0, rng.standard_normal((B, L, shape.Hv)))
    b = scipy.special.expit(rng.standard_normal((B, L, shape.Hv)))
    st = conv_std * rng.standard_normal((B, shape.D, shape.K - 1))
    S0 = s0_std * rng.standard_normal((B, shape.Hv, shape.dk, shape.dv))
    return x, g, b, w, st, S0


def pin_layer_composition():
    shape = gi.TINY_GQA
    p = oracle.OracleParams.of(shape)
    x, g, b, w, st, S0 = _layer_case(shape, 2, 9, 41)
    res = oracle.gdn_forward(p, x, g, b, w, st, S0)
    q, k, v = oracle.front_end(p, x, w, st)
    for bb in range(2):
        for h in range(shape.Hv):
            o, S = oracle.delta_rule(q[bb, :, h], k[bb, :, h], v[bb, :, h], g[bb, :, h], b[bb, :, h], S0[bb, h])
            assert np.array_equal(o, res["o"][bb, :, h]) and np.array_equal(S, res["S"][bb, h])
    _, cout = oracle.conv1d_silu(p, x, w, st)
    assert np.array_equal(cout, res["conv_out"])


def pin_layer_carry_invariants():
    shape = gi.TINY_GQA
    p = oracle.OracleParams.of(shape)
    B, L = 2, 11
    x, g, b, w, st, S0 = _layer_case(shape, B, L, 42)
    full = oracle.gdn_forward(p, x, g, b, w, st, S0, snapshots=True)
    # split calls == one call
    r1 = oracle.gdn_forward(p, x[:, :, :4], g[:, :4], b[:, :4], w, st, S0)
    r2 = oracle.gdn_forward(p, x[:, :, 4:], g[:, 4:], b[:, 4:], w, r1["conv_out"], r1["S"])
    assert _rel(np.concatenate([r1["o"], r2["o"]], axis=1), full["o"]) < 1e-13
    assert _rel(r2["S"], full["S"]) < 1e-13
    assert np.array_equal(r2["conv_out"], full["conv_out"])
    # one token at a time (decode) == one call; snapshots are the per-token states
    S, cs = S0.copy(), st.copy()
    for t in range(L):
        r = oracle.gdn_forward(p, x[:, :, t:t + 1], g[:, t:t + 1], b[:, t:t + 1], w, cs, S)
        S, cs = r["S"], r["conv_out"]
        assert _rel(r["o"][:, 0], full["o"][:, t]) < 1e-13
        assert _rel(S, full["snap"][:, t]) < 1e-13
    assert _rel(S, full["S"]) < 1e-13
    # ragged packing == separate calls
    lens = [3, 0, 5, 1]
    cu = gi.cu_seqlens(lens)
    N = len(lens)
    rng = np.random.default_rng(43)
    xp = rng.standard_normal((1, shape.D, int(cu[-1])))
    gp = -np.logaddexp(0, rng.standard_normal((1, int(cu[-1]), shape.Hv)))
    bp = scipy.special.expit(rng.standard_normal((1, int(cu[-1]), shape.Hv)))
    stp = rng.standard_normal((N, shape.D, shape.K - 1))
    S0p = 0.1 * rng.standard_normal((N, shape.Hv, shape.dk, shape.dv))
    packed = oracle.gdn_forward(p, xp, gp, bp, w, stp, S0p, cu_seqlens=cu)
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        sep = oracle.gdn_forward(p, xp[:, :, s:e], gp[:, s:e], bp[:, s:e], w, stp[n:n + 1], S0p[n:n + 1])
        assert np.array_equal(sep["o"][0], packed["o"][0, s:e])
        assert np.array_equal(sep["S"][0], packed["S"][n])
        assert np.array_equal(sep["conv_out"][0], packed["conv_out"][n])


def pin_verify_commit():
    shape = gi.TINY_GQA
    p = oracle.OracleParams.of(shape)
    B, T = 4, 4
    x, g, b, w, st, S0 = _layer_case(shape, B, T, 44)
    full = oracle.gdn_forward(p, x, g, b, w, st, S0, snapshots=True)
    acc = np.array([0, 1, 2, 3], np.int32)
    S_out, c_out = oracle.verify_commit(p, acc, x, st, full["snap"])
    for bb in range(B):
        a = int(acc[bb])
        r = oracle.gdn_forward(p, x[bb:bb + 1, :, :a + 1], g[bb:bb + 1, :a + 1], b[bb:bb + 1, :a + 1],
                               w, st[bb:bb + 1], S0[bb:bb + 1])
        assert np.array_equal(S_out[bb], full["snap"][bb, a])
        assert _rel(S_out[bb], r["S"][0]) < 1e-13
        assert np.array_equal(c_out[bb], r["conv_out"][0])


# ---------------------------------------------------------------------------
# gate/beta parameterisation and gated RMSNorm
# ---------------------------------------------------------------------------
def pin_gate_beta():
    import torch
    rng = np.random.default_rng(51)
    Hv = 6
    a = 3.0 * rng.standard_normal((5, Hv))
    b = 3.0 * rng.standard_normal((5, Hv))
    A_log = rng.standard_normal(Hv)
    dt_bias = rng.standard_normal(Hv)
    g, be = oracle.gate_beta(a, b, A_log, dt_bias)
    ta = torch.from_numpy(a)
    ref_g = (-torch.exp(torch.from_numpy(A_log)) * torch.nn.functional.softplus(ta + torch.from_numpy(dt_bias))).numpy()
    ref_b = torch.sigmoid(torch.from_numpy(b)).numpy()
    assert _rel(g, ref_g) < 1e-14 and _rel(be, ref_b) < 1e-14
    assert np.all(g <= 0) and np.all((be > 0) & (be < 1))
    # closed forms: a + dt_bias = 0 gives softplus = ln 2; A_log = 0 gives a unit factor
    g0, b0 = oracle.gate_beta(-np.ones((1, 2)), np.zeros((1, 2)), np.zeros(2), np.ones(2))
    assert np.allclose(g0, -math.log(2.0), rtol=0, atol=1e-15) and np.allclose(b0, 0.5, rtol=0, atol=1e-16)
    _, bp = oracle.gate_beta(a, b, A_log, dt_bias)
    _, bm = oracle.gate_beta(a, -b, A_log, dt_bias)
    assert np.allclose(bp + bm, 1.0, rtol=0, atol=1e-15)


def pin_gated_rmsnorm():
    import torch
    rng = np.random.default_rng(52)
    dv = 16
    x = rng.standard_normal((7, 3, dv))
    z = rng.standard_normal((7, 3, dv))
    w = 1.0 + 0.2 * rng.standard_normal(dv)
    eps = 1e-6
    out = oracle.gated_rmsnorm(x, z, w, eps)
    tx, tz = torch.from_numpy(x), torch.from_numpy(z)
    ref = (torch.nn.functional.rms_norm(tx, (dv,), torch.from_numpy(w), eps) * torch.nn.functional.silu(tz)).numpy()
    assert _rel(out, ref) < 1e-14
    # scale invariance (up to eps) and a zero gate
    assert _rel(oracle.gated_rmsnorm(4.0 * x, z, w, 0.0), oracle.gated_rmsnorm(x, z, w, 0.0)) < 1e-14
    assert np.array_equal(oracle.gated_rmsnorm(x, np.zeros_like(z), w, eps), np.zeros_like(x))


ALL_PINS = [
    pin_hand_worked, pin_rational_brute_force, pin_kronecker_form, pin_chunked_form,
    pin_closed_forms, pin_lms_and_norm_bound, pin_conv_library, pin_conv_onehot_and_carry,
    pin_front_end_mapping_and_norms, pin_gqa_end_to_end_probe, pin_layer_composition,
    pin_layer_carry_invariants, pin_verify_commit, pin_gate_beta, pin_gated_rmsnorm,
]
