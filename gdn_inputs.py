"""Seeded synthetic inputs for the Gated DeltaNet layer.

This module is shared by the fp64 oracle side (tests, cpu baseline) and the
HIP side (tests, bench). It holds none of the layer's arithmetic: it only
draws random tensors with the distributions and shapes of the workloads and
rounds them to the storage precision.

Every tensor comes from its own stream ``numpy.random.default_rng([seed,
tensor_id, *extra])`` so that any tensor can be regenerated on its own.

Value distributions (the tiny fp32 case and all bf16 cases use the same ones):
  qkv          ~ N(0, 1)                      [B, D, L]
  conv_weight  ~ N(0, 0.5^2)  (std 0.5)       [D, 1, K]
  gate         = -softplus(N(0, 1))  (<= 0)   [B, L, Hv]
  beta         = sigmoid(N(0, 1))             [B, L, Hv]
  S0           ~ N(0, 0.1^2) or zero          [N, Hv, dk, dv]  (always fp32)
  conv_state0  ~ N(0, 1) or zero              [N, D, K-1]

Inputs of the optional prologue/epilogue fusions:
  a_raw, b_raw ~ N(0, 1)                      [B, L, Hv]  (raw gate/beta projections)
  A_log        = log(U(1, 16))                [Hv]
  dt_bias      = softplus^-1(dt), log10(dt) ~ U(-3, -1)   [Hv]
  z            ~ N(0, 1)                      [B, L, Hv, dv]
  norm_weight  ~ 1 + N(0, 0.1^2)              [dv]

Values are drawn in float64 and rounded once, by round-to-nearest-even, to the
storage type (bf16 or fp32). All arrays are returned as float32 numpy arrays
whose values are exactly representable in the storage type, so both sides see
identical numbers: the oracle widens them to float64, the GPU side stores them
as bf16 (or fp32) bits.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# tensor ids of the per-tensor random streams
TID_QKV, TID_W, TID_GATE, TID_BETA, TID_S0, TID_CONV0, TID_ACCEPT, TID_LENS = range(8)
TID_A_RAW, TID_B_RAW, TID_A_LOG, TID_DT_BIAS, TID_Z, TID_NORM_W = range(8, 14)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits) by round-to-nearest-even.

    Works on the float64 bit pattern: drop the low 45 of the 52 stored mantissa
    bits with RNE. Carries into the exponent are handled by the integer add.
    Returned as float32 (exact, since every bf16 value is an fp32 value).
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = a.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64).astype(np.float32)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def _rng(seed: int, tid: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid, *extra])


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


@dataclasses.dataclass(frozen=True)
class Shape:
    """Layer shape: heads, head dims, conv taps."""
    Hk: int
    Hv: int
    dk: int
    dv: int
    K: int = 4

    @property
    def D(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


def qkv(shape: Shape, B: int, L: int, seed: int, dtype: str, step: int | None = None) -> np.ndarray:
    extra = () if step is None else (step,)
    return round_to(_rng(seed, TID_QKV, *extra).standard_normal((B, shape.D, L)), dtype)


def conv_weight(shape: Shape, seed: int, dtype: str) -> np.ndarray:
    return round_to(_rng(seed, TID_W).normal(0.0, 0.5, (shape.D, 1, shape.K)), dtype)


def gate(shape: Shape, B: int, L: int, seed: int, dtype: str, step: int | None = None) -> np.ndarray:
    extra = () if step is None else (step,)
    return round_to(-_softplus(_rng(seed, TID_GATE, *extra).standard_normal((B, L, shape.Hv))), dtype)


def beta(shape: Shape, B: int, L: int, seed: int, dtype: str, step: int | None = None) -> np.ndarray:
    extra = () if step is None else (step,)
    return round_to(_sigmoid(_rng(seed, TID_BETA, *extra).standard_normal((B, L, shape.Hv))), dtype)


def state0(shape: Shape, N: int, seed: int, std: float) -> np.ndarray:
    if std == 0.0:
        return np.zeros((N, shape.Hv, shape.dk, shape.dv), np.float32)
    return round_to(_rng(seed, TID_S0).normal(0.0, std, (N, shape.Hv, shape.dk, shape.dv)), "f32")


def conv_state0(shape: Shape, N: int, seed: int, std: float, dtype: str) -> np.ndarray:
    if std == 0.0:
        return np.zeros((N, shape.D, shape.K - 1), np.float32)
    return round_to(_rng(seed, TID_CONV0).normal(0.0, std, (N, shape.D, shape.K - 1)), dtype)


def a_raw(shape: Shape, B: int, L: int, seed: int, dtype: str, step: int | None = None) -> np.ndarray:
    extra = () if step is None else (step,)
    return round_to(_rng(seed, TID_A_RAW, *extra).standard_normal((B, L, shape.Hv)), dtype)


def b_raw(shape: Shape, B: int, L: int, seed: int, dtype: str, step: int | None = None) -> np.ndarray:
    extra = () if step is None else (step,)
    return round_to(_rng(seed, TID_B_RAW, *extra).standard_normal((B, L, shape.Hv)), dtype)


def a_log(shape: Shape, seed: int, dtype: str) -> np.ndarray:
    return round_to(np.log(_rng(seed, TID_A_LOG).uniform(1.0, 16.0, shape.Hv)), dtype)


def dt_bias(shape: Shape, seed: int, dtype: str) -> np.ndarray:
    dt = 10.0 ** _rng(seed, TID_DT_BIAS).uniform(-3.0, -1.0, shape.Hv)
    return round_to(dt + np.log(-np.expm1(-dt)), dtype)   # the x with log(1 + e^x) = dt


def z_gate(shape: Shape, B: int, L: int, seed: int, dtype: str, step: int | None = None) -> np.ndarray:
    extra = () if step is None else (step,)
    return round_to(_rng(seed, TID_Z, *extra).standard_normal((B, L, shape.Hv, shape.dv)), dtype)


def norm_weight(shape: Shape, seed: int, dtype: str) -> np.ndarray:
    return round_to(1.0 + _rng(seed, TID_NORM_W).normal(0.0, 0.1, shape.dv), dtype)


def accept_len(B: int, T: int, seed: int) -> np.ndarray:
    """Accepted drafted tokens per sequence, uniform on the integers 0..T-1 (inclusive)."""
    return _rng(seed, TID_ACCEPT).integers(0, T, size=B, endpoint=False).astype(np.int32)


def seq_lens(N: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Ragged sequence lengths, uniform on the integers lo..hi (inclusive)."""
    return _rng(seed, TID_LENS).integers(lo, hi, size=N, endpoint=True).astype(np.int32)


def cu_seqlens(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    return cu.astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads. seed = 1000 + index.
# ---------------------------------------------------------------------------
TINY = Shape(Hk=2, Hv=2, dk=16, dv=16, K=4)          # D = 96
QWEN = Shape(Hk=16, Hv=32, dk=128, dv=128, K=4)      # D = 8192
TINY_GQA = Shape(Hk=2, Hv=4, dk=16, dv=16, K=4)      # extra GQA variant of the tiny case


@dataclasses.dataclass
class Workload:
    name: str
    shape: Shape
    dtype: str
    seed: int


WORKLOADS = {
    0: Workload("tiny_fp32_B1_L64_d16", TINY, "f32", 1000),
    1: Workload("decode_B64_Hk16_Hv32_d128_256steps", QWEN, "bf16", 1001),
    2: Workload("prefill_B1_L4096_Hk16_Hv32_d128_chunk64", QWEN, "bf16", 1002),
    3: Workload("ragged_prefill_8seqs_L512-8192_Hk16_Hv32_d128", QWEN, "bf16", 1003),
    4: Workload("verify_B128_T4_Hk16_Hv32_d128", QWEN, "bf16", 1004),
}

DECODE_B, DECODE_STEPS = 64, 256
PREFILL_L = 4096
RAGGED_N, RAGGED_LO, RAGGED_HI = 8, 512, 8192
VERIFY_B, VERIFY_T = 128, 4
