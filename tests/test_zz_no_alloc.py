"""gdn_prefill_ex_noalloc (workspace in the library's static device scratch) against
gdn_prefill_ex with a caller workspace, through the C ABI: the same kernels on the same
inputs, so the outputs, final states and conv windows agree bit for bit. Two calls in a
row on the one scratch array, the second smaller than the first (a segmented 1024-token
prompt, then three packed prompts with both fusions), so that the second call runs over
what the first left in the scratch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_sequence_amd as gdn
from gpu_cases import dev, layer_inputs, params

pytestmark = pytest.mark.gpu
SH = gi.QWEN


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load()


def _both(inp, cu=None, fusion=None):
    p = params(SH, "bf16")
    B, _, L = inp["qkv"].shape
    N = inp["S0"].shape[0]
    args = [dev(inp["qkv"], "bf16"), dev(inp["gate"], "bf16"), dev(inp["beta"], "bf16"), dev(inp["w"], "bf16"),
            dev(inp["conv0"], "bf16")]
    cud = None if cu is None else dev(np.asarray(cu, np.int32))
    out = []
    for noalloc in (True, False):
        S = dev(inp["S0"])
        o = torch.full((B, L, SH.Hv, SH.dv), float("nan"), device="cuda")
        cout = torch.zeros_like(args[4])
        if noalloc:
            gdn.gdn_prefill_ex_noalloc(p, fusion, *args, cout, S, o, cu_seqlens=cud)
        else:
            ws = gdn.prefill_workspace(p, B, L, N)
            gdn.gdn_prefill_ex(p, fusion, *args, cout, S, o, ws, cu_seqlens=cud)
        torch.cuda.synchronize()
        out.append((o, S, cout))
    return out


def test_noalloc_prefill_two_calls_match_the_workspace_call():
    print("noalloc prefill: 1024-token prompt (4 carry segments)", flush=True)
    inp = layer_inputs(SH, 1, 1024, 61, "bf16", s0_std=0.1, conv_std=1.0)
    (o1, S1, c1), (o2, S2, c2) = _both(inp)
    assert not torch.isnan(o1).any()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)

    print("noalloc prefill: 3 packed prompts (300 tokens), prologue + epilogue", flush=True)
    lens = [100, 7, 193]
    cu = gi.cu_seqlens(lens)
    inp = layer_inputs(SH, 1, int(cu[-1]), 62, "bf16", N=len(lens), s0_std=0.1, conv_std=1.0)
    L = int(cu[-1])
    fu = gdn.GdnFusion(dev(gi.a_log(SH, 62, "bf16"), "bf16"), dev(gi.dt_bias(SH, 62, "bf16"), "bf16"),
                       dev(gi.z_gate(SH, 1, L, 62, "bf16"), "bf16"), dev(gi.norm_weight(SH, 62, "bf16"), "bf16"),
                       1e-6)
    inp["gate"], inp["beta"] = gi.a_raw(SH, 1, L, 62, "bf16"), gi.b_raw(SH, 1, L, 62, "bf16")
    (o1, S1, c1), (o2, S2, c2) = _both(inp, cu=cu, fusion=fu)
    assert not torch.isnan(o1).any()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)


def test_noalloc_prefill_refuses_prompts_beyond_its_scratch():
    p = params(SH, "bf16")
    L = 8192
    assert gdn.gdn_prefill_workspace_size(p, 1, L, 1) > (128 << 20)
    inp = layer_inputs(SH, 1, L, 63, "bf16")
    args = [dev(inp[k], "bf16") for k in ("qkv", "gate", "beta", "w", "conv0")]
    S = dev(inp["S0"])
    o = torch.empty((1, L, SH.Hv, SH.dv), device="cuda")
    with pytest.raises(gdn.GdnError, match="GDN_ERR_TOO_LARGE"):
        gdn.gdn_prefill_ex_noalloc(p, None, *args, torch.empty_like(args[4]), S, o)
