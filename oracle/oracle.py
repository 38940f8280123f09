"""numpy/ctypes wrapper of the fp64 C oracle (TEST INFRASTRUCTURE ONLY).

Every function widens its inputs to float64, calls the C routine of the same
name in gdn_oracle.c and returns float64 arrays. The C file documents which
passage of "MNN Model Support: Qwen3.5" (§1.2 steps 1-5, §1.3, §1.4) each
routine follows.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")

MUTATIONS = {
    "no_decay_before_predict": 1,
    "delta_sign": 2,
    "gqa_tiled": 3,
    "out_pre_write": 4,
    "scale_before_norm": 5,
    "conv_reversed": 6,
    "k_not_normed": 7,
    "conv_state_shift": 8,
    "predict_transposed": 9,
    "no_beta": 10,
    "qk_swapped": 11,
    "no_silu": 12,
    "decay_after_write": 13,
    "gate_sign": 14,
    "rms_sum": 15,
    "rms_sigmoid_gate": 16,
}


def build_oracle(force: bool = True) -> str:
    """Compile gdn_oracle.c with gcc into libgdn_oracle.so (next to the source)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_oracle(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.orc_set_mutation.argtypes = [I]
        lib.orc_get_mutation.restype = I
        lib.orc_delta_rule.argtypes = [I, I, I, P, P, P, P, P, P, P, P]
        lib.orc_conv1d_silu.argtypes = [P, I, I, P, P, P, P, P, P, I, I]
        lib.orc_front_end.argtypes = [P, I, I, P, P, P, P, I, P, P, P]
        lib.orc_gdn_forward.argtypes = [P, I, I, P, P, P, P, P, P, P, P, P, P, I, P, I]
        lib.orc_verify_commit.argtypes = [P, I, I, P, P, P, P, P, P]
        lib.orc_gate_beta.argtypes = [ctypes.c_int64, I, P, P, P, P, P, P]
        lib.orc_gated_rmsnorm.argtypes = [ctypes.c_int64, I, P, P, P, ctypes.c_double, P]
        for f in (lib.orc_delta_rule, lib.orc_conv1d_silu, lib.orc_front_end,
                  lib.orc_gdn_forward, lib.orc_verify_commit, lib.orc_gate_beta,
                  lib.orc_gated_rmsnorm):
            f.restype = I
        _lib = lib
    return _lib


class _CParams(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int), ("num_v_heads", ctypes.c_int),
                ("head_k_dim", ctypes.c_int), ("head_v_dim", ctypes.c_int),
                ("conv_k", ctypes.c_int), ("use_qk_l2norm", ctypes.c_int),
                ("eps", ctypes.c_double)]


@dataclasses.dataclass(frozen=True)
class OracleParams:
    """LinearAttentionParam (page §1.4) plus the conv width and the L2-norm epsilon."""
    Hk: int
    Hv: int
    dk: int
    dv: int
    K: int = 4
    use_qk_l2norm: bool = True
    eps: float = 1e-6

    @property
    def D(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv

    def c(self) -> _CParams:
        return _CParams(self.Hk, self.Hv, self.dk, self.dv, self.K, int(self.use_qk_l2norm), self.eps)

    @staticmethod
    def of(shape, **kw) -> "OracleParams":
        return OracleParams(shape.Hk, shape.Hv, shape.dk, shape.dv, shape.K, **kw)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(st, name):
    if st != 0:
        raise ValueError(f"oracle {name} rejected its arguments (status {st})")


def set_mutation(m: int) -> None:
    _load().orc_set_mutation(int(m))


@contextlib.contextmanager
def mutation(name: str):
    """Plant one known mistake in the oracle for the duration of the block."""
    set_mutation(MUTATIONS[name])
    try:
        yield
    finally:
        set_mutation(0)


def delta_rule(q, k, v, g, beta, S0, snapshots: bool = False):
    """Step 5 for one head: q, k [L,dk]; v [L,dv]; g, beta [L]; S0 [dk,dv].

    Returns (o [L,dv], S_final [dk,dv]) or (o, S_final, snap [L,dk,dv])."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    S = _f64(S0).copy()
    L, dk = q.shape
    dv = v.shape[1]
    o = np.zeros((L, dv))
    snap = np.zeros((L, dk, dv)) if snapshots else None
    _check(_load().orc_delta_rule(L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(S), _ptr(o), _ptr(snap)), "delta_rule")
    return (o, S, snap) if snapshots else (o, S)


def _segments(B, L, cu_seqlens, N):
    if cu_seqlens is None:
        return None, B
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    return cu, (len(cu) - 1 if N is None else N)


def conv1d_silu(p: OracleParams, x, w, conv_in, cu_seqlens=None, N=None, nthreads=None):
    """Step 1 alone. x [B,D,L], w [D,1,K], conv_in [N,D,K-1] -> (y [B,D,L], conv_out)."""
    x, w, conv_in = map(_f64, (x, w, conv_in))
    B, D, L = x.shape
    cu, N = _segments(B, L, cu_seqlens, N)
    y = np.zeros_like(x)
    conv_out = np.zeros((N, D, p.K - 1))
    pc = p.c()
    _check(_load().orc_conv1d_silu(ctypes.byref(pc), B, L, _ptr(x), _ptr(w), _ptr(conv_in),
                                   _ptr(conv_out), _ptr(y), _ptr(cu), N,
                                   nthreads or default_threads()), "conv1d_silu")
    return y, conv_out


def front_end(p: OracleParams, x, w, conv_in, cu_seqlens=None, N=None):
    """Steps 1-4. Returns q_hat, k_hat [B,L,Hv,dk] (expanded to V heads), v [B,L,Hv,dv]."""
    x, w, conv_in = map(_f64, (x, w, conv_in))
    B, D, L = x.shape
    cu, N = _segments(B, L, cu_seqlens, N)
    q = np.zeros((B, L, p.Hv, p.dk))
    k = np.zeros((B, L, p.Hv, p.dk))
    v = np.zeros((B, L, p.Hv, p.dv))
    pc = p.c()
    _check(_load().orc_front_end(ctypes.byref(pc), B, L, _ptr(x), _ptr(w), _ptr(conv_in),
                                 _ptr(cu), N, _ptr(q), _ptr(k), _ptr(v)), "front_end")
    return q, k, v


def gdn_forward(p: OracleParams, x, gate, beta, w, conv_in, S0, cu_seqlens=None, N=None,
                snapshots: bool = False, unit_mask=None, nthreads=None):
    """Whole layer (steps 1-5). x [B,D,L]; gate, beta [B,L,Hv]; w [D,1,K];
    conv_in [N,D,K-1]; S0 [N,Hv,dk,dv].

    Returns dict(o [B,L,Hv,dv], S [N,Hv,dk,dv], conv_out [N,D,K-1], snap [B,L,Hv,dk,dv] or None).
    With unit_mask [N,Hv] (bool) only the selected (sequence, head) units are computed;
    the others keep S0 and a zero output."""
    x, gate, beta, w, conv_in = map(_f64, (x, gate, beta, w, conv_in))
    B, D, L = x.shape
    cu, N = _segments(B, L, cu_seqlens, N)
    S = _f64(S0).copy()
    o = np.zeros((B, L, p.Hv, p.dv))
    conv_out = np.zeros((N, D, p.K - 1))
    snap = np.zeros((B, L, p.Hv, p.dk, p.dv)) if snapshots else None
    mask = None
    if unit_mask is not None:
        mask = np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8).reshape(N * p.Hv))
    pc = p.c()
    _check(_load().orc_gdn_forward(ctypes.byref(pc), B, L, _ptr(x), _ptr(gate), _ptr(beta),
                                   _ptr(w), _ptr(conv_in), _ptr(conv_out), _ptr(S), _ptr(o),
                                   _ptr(snap), _ptr(cu), N, _ptr(mask),
                                   nthreads or default_threads()), "gdn_forward")
    return {"o": o, "S": S, "conv_out": conv_out, "snap": snap}


def verify_commit(p: OracleParams, accept_len, x, conv_in, snap):
    """Keep the snapshot after token accept_len[b] and roll the conv window to match.
    x [B,D,T]; conv_in [B,D,K-1]; snap [B,T,Hv,dk,dv] -> (S_out [B,Hv,dk,dv], conv_out)."""
    x, conv_in, snap = map(_f64, (x, conv_in, snap))
    acc = np.ascontiguousarray(np.asarray(accept_len, dtype=np.int32))
    B, D, T = x.shape
    S_out = np.zeros((B, p.Hv, p.dk, p.dv))
    conv_out = np.zeros((B, D, p.K - 1))
    pc = p.c()
    _check(_load().orc_verify_commit(ctypes.byref(pc), B, T, _ptr(acc), _ptr(x), _ptr(conv_in),
                                     _ptr(snap), _ptr(conv_out), _ptr(S_out)), "verify_commit")
    return S_out, conv_out


def gate_beta(a, b, A_log, dt_bias):
    """gate = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b). a, b [..., Hv]; A_log, dt_bias [Hv]."""
    a, b, A_log, dt_bias = map(_f64, (a, b, A_log, dt_bias))
    Hv = A_log.shape[0]
    n = a.size // Hv
    gate = np.zeros_like(a)
    beta = np.zeros_like(b)
    _check(_load().orc_gate_beta(n, Hv, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(gate),
                                 _ptr(beta)), "gate_beta")
    return gate, beta


def gated_rmsnorm(x, z, weight, eps):
    """weight * x * rsqrt(mean(x^2) + eps) * silu(z) over the last dimension."""
    x, z, weight = map(_f64, (x, z, weight))
    dv = x.shape[-1]
    out = np.zeros_like(x)
    _check(_load().orc_gated_rmsnorm(x.size // dv, dv, _ptr(x), _ptr(z), _ptr(weight), float(eps),
                                     _ptr(out)), "gated_rmsnorm")
    return out
