"""Shared helpers of the GPU parity tests: seeded inputs as numpy (for the oracle)
and as device tensors (for the HIP path), and the error metric.

Tolerances: max|gpu - oracle| / max|oracle| per output tensor is at most 1e-5
with fp32 inputs and 2e-3 with bf16 inputs (fp32 state and accumulation on the
GPU, fp64 in the oracle). Raw conv-state copies and index work are compared
bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import gdn_inputs as gi
import linear_attention_sequence_amd as gdn
import oracle

TOL = {"f32": 1e-5, "bf16": 2e-3}


def rel_err(gpu, ref) -> float:
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(r))) if r.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(g))) if g.size else 0.0
    return float(np.max(np.abs(g - r)) / den)


def params(shape: gi.Shape, dtype: str, use_l2=True) -> gdn.GdnParams:
    return gdn.GdnParams(shape.Hk, shape.Hv, shape.dk, shape.dv, shape.K, use_l2, 1e-6,
                         gdn.GDN_BF16 if dtype == "bf16" else gdn.GDN_F32)


def oparams(shape: gi.Shape, use_l2=True) -> oracle.OracleParams:
    return oracle.OracleParams.of(shape, use_qk_l2norm=use_l2)


def dev(a, dtype: str | None = None):
    """numpy -> device tensor; bf16 values are exact (inputs are pre-rounded)."""
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.contiguous()


def layer_inputs(shape: gi.Shape, B: int, L: int, seed: int, dtype: str, N=None,
                 s0_std=0.0, conv_std=0.0, step=None):
    """qkv, gate, beta, conv_weight, conv_state0, S0 for a (B, L) call."""
    N = B if N is None else N
    return dict(
        qkv=gi.qkv(shape, B, L, seed, dtype, step=step),
        gate=gi.gate(shape, B, L, seed, dtype, step=step),
        beta=gi.beta(shape, B, L, seed, dtype, step=step),
        w=gi.conv_weight(shape, seed, dtype),
        conv0=gi.conv_state0(shape, N, seed, conv_std, dtype),
        S0=gi.state0(shape, N, seed, s0_std),
    )


def run_prefill(shape, dtype, inp, cu=None, qkv_offset=0, o_fill=0.0):
    """qkv_offset > 0 places qkv that many elements into a larger buffer (so its address
    is only element-aligned); o starts filled with o_fill."""
    p = params(shape, dtype)
    B, D, L = inp["qkv"].shape
    N = inp["S0"].shape[0]
    S = dev(inp["S0"])
    o = torch.full((B, L, shape.Hv, shape.dv), o_fill, dtype=torch.float32, device="cuda")
    cout = torch.zeros_like(dev(inp["conv0"], dtype))
    ws = gdn.prefill_workspace(p, B, L, N)
    x = dev(inp["qkv"], dtype)
    if qkv_offset:
        buf = torch.zeros(x.numel() + qkv_offset, dtype=x.dtype, device="cuda")
        buf[qkv_offset:].copy_(x.reshape(-1))
        x = buf[qkv_offset:].view(x.shape)
    gdn.gdn_prefill(p, x, dev(inp["gate"], dtype), dev(inp["beta"], dtype),
                    dev(inp["w"], dtype), dev(inp["conv0"], dtype), cout, S, o, ws,
                    cu_seqlens=None if cu is None else dev(np.asarray(cu, np.int32)))
    torch.cuda.synchronize()
    return {"o": o, "S": S, "conv_out": cout}
