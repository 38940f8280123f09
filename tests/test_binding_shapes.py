"""The Python binding rejects tensors whose shape differs from the one the call derives
(from the params and the leading tensor) with ValueError, before any pointer is taken
or anything is launched. Runs on the CPU: the tensors live in host memory, so a call
that passed every shape check would stop at the device check instead."""
import pytest
import torch

import linear_attention_sequence_amd as gdn

P = gdn.GdnParams(2, 4, 16, 16, 4, True, 1e-6, gdn.GDN_BF16)   # D = 2*2*16 + 4*16 = 128
B, L, T, N = 2, 5, 3, 2
D, Hv, d = P.D, 4, 16
bf, f32 = torch.bfloat16, torch.float32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def decode_args(**over):
    a = dict(qkv=z(B, D, 1), gate=z(B, 1, Hv), beta=z(B, 1, Hv), conv_weight=z(D, 1, 4),
             conv_state_in=z(B, D, 3), conv_state_out=z(B, D, 3), S=z(B, Hv, d, d, dtype=f32),
             o=z(B, 1, Hv, d, dtype=f32))
    a.update(over)
    return a


def verify_args(**over):
    a = dict(qkv=z(B, D, T), gate=z(B, T, Hv), beta=z(B, T, Hv), conv_weight=z(D, 1, 4),
             conv_state_in=z(B, D, 3), S_in=z(B, Hv, d, d, dtype=f32),
             S_snap=z(B, T, Hv, d, d, dtype=f32), o=z(B, T, Hv, d, dtype=f32))
    a.update(over)
    return a


def prefill_args(**over):
    a = dict(qkv=z(1, D, L), gate=z(1, L, Hv), beta=z(1, L, Hv), conv_weight=z(D, 1, 4),
             conv_state_in=z(N, D, 3), conv_state_out=z(N, D, 3), S=z(N, Hv, d, d, dtype=f32),
             o=z(1, L, Hv, d, dtype=f32), workspace=z(16, dtype=torch.uint8),
             cu_seqlens=torch.tensor([0, 2, 5], dtype=torch.int32))
    a.update(over)
    return a


def _raises_shape(fn, name, **kw):
    with pytest.raises(ValueError, match=rf"^{name} (has shape|must have)"):
        fn(P, **kw)


@pytest.mark.parametrize("name,bad", [
    ("gate", z(B, 1, Hv - 1)), ("beta", z(B, 2, Hv)), ("conv_weight", z(D, 1, 3)),
    ("conv_state_in", z(B + 1, D, 3)), ("conv_state_out", z(B, D, 2)),
    ("S", z(B, Hv, d, d - 1, dtype=f32)), ("o", z(B, 1, Hv, d - 4, dtype=f32)),
])
def test_decode_shapes(name, bad):
    _raises_shape(gdn.gdn_decode_step, name, **decode_args(**{name: bad}))


def test_decode_fusion_shapes():
    fu = gdn.GdnFusion(z(Hv), z(Hv), z(B, 1, Hv, d), z(d + 1), 1e-6)
    with pytest.raises(ValueError, match="^norm_weight has shape"):
        gdn.gdn_decode_step_ex(P, fu, **decode_args())
    fu = gdn.GdnFusion(z(Hv), z(Hv), z(B, 2, Hv, d), z(d), 1e-6)
    with pytest.raises(ValueError, match="^z has shape"):
        gdn.gdn_decode_step_ex(P, fu, **decode_args())


@pytest.mark.parametrize("name,bad", [
    ("S_snap", z(B, T - 1, Hv, d, d, dtype=f32)), ("S_in", z(B, Hv, d, 1, dtype=f32)),
    ("o", z(B, T, Hv, d - 1, dtype=f32)), ("gate", z(B, T - 1, Hv)),
])
def test_verify_shapes(name, bad):
    _raises_shape(gdn.gdn_verify_block, name, **verify_args(**{name: bad}))


def test_verify_slots_and_commit_shapes():
    a = verify_args()
    a.pop("S_in")
    slot = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="^slot has shape"):
        gdn.gdn_verify_block_slots(P, None, S_prev=z(B, 2, Hv, d, d, dtype=f32), slot=slot[:1], **a)
    with pytest.raises(ValueError, match="^S_prev has shape"):
        gdn.gdn_verify_block_slots(P, None, S_prev=z(B, 2, Hv, d, 1, dtype=f32), slot=slot, **a)
    c = dict(accept_len=slot, qkv=z(B, D, T), conv_state_in=z(B, D, 3), S_snap=z(B, T, Hv, d, d, dtype=f32),
             conv_state_out=z(B, D, 3), S_out=z(B, Hv, d, d, dtype=f32))
    with pytest.raises(ValueError, match="^accept_len has shape"):
        gdn.gdn_verify_commit(P, **{**c, "accept_len": slot[:1]})
    with pytest.raises(ValueError, match="^S_out has shape"):
        gdn.gdn_verify_commit(P, **{**c, "S_out": z(B - 1, Hv, d, d, dtype=f32)})


@pytest.mark.parametrize("name,bad", [
    ("o", z(1, L - 1, Hv, d, dtype=f32)), ("S", z(N, Hv, d, d - 1, dtype=f32)),
    ("conv_state_out", z(N - 1, D, 3)), ("gate", z(1, L, Hv + 1)),
    ("cu_seqlens", torch.tensor([0, 5], dtype=torch.int32)),
])
def test_prefill_shapes(name, bad):
    _raises_shape(gdn.gdn_prefill, name, **prefill_args(**{name: bad}))


def test_conv_shapes():
    with pytest.raises(ValueError, match="^y has shape"):
        gdn.gdn_conv1d_silu(P, z(B, D, L), z(D, 1, 4), z(B, D, 3), z(B, D, 3), z(B, D, L - 1, dtype=f32))


def test_well_shaped_host_tensors_stop_at_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        gdn.gdn_decode_step(P, **decode_args())
    with pytest.raises(ValueError, match="GPU"):
        gdn.gdn_prefill(P, **prefill_args())
