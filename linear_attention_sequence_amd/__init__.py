"""Python binding of libgdn.so, the MI355X Gated DeltaNet layer (include/gdn.h).

Argument marshalling only: each function checks that the torch tensors it is
given have the dtype and the exact shape the call derives from the params and
the leading tensor (ValueError otherwise, before anything is launched), that
they are contiguous device tensors, reads the sizes off their shapes and passes
raw pointers plus the current HIP stream to the C entry point of the same name. All arithmetic runs in the HIP kernels of libgdn.so;
there is no fallback. If the library is missing the import still succeeds
(so that `build()` can run) but every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE",
          4: "GDN_ERR_UNSUPPORTED", 5: "GDN_ERR_ALIAS", 6: "GDN_ERR_WORKSPACE",
          7: "GDN_ERR_LAUNCH", 8: "GDN_ERR_ALIGN", 9: "GDN_ERR_TOO_LARGE"}

# every symbol include/gdn.h declares
EXPORTS = ("gdn_status_string", "gdn_version", "gdn_conv1d_silu", "gdn_decode_step",
           "gdn_verify_block", "gdn_verify_commit", "gdn_prefill_workspace_size", "gdn_prefill",
           "gdn_decode_step_ex", "gdn_verify_block_ex", "gdn_prefill_ex", "gdn_verify_block_slots",
           "gdn_prefill_ex_noalloc")


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


class _CParams(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
                ("conv_kernel", ctypes.c_int32), ("use_qk_l2norm", ctypes.c_int32),
                ("l2norm_eps", ctypes.c_float), ("in_dtype", ctypes.c_int32)]


@dataclasses.dataclass(frozen=True)
class GdnParams:
    """gdn_params: LinearAttentionParam plus conv width, L2-norm epsilon and input dtype."""
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_kernel: int = 4
    use_qk_l2norm: bool = True
    l2norm_eps: float = 1e-6
    in_dtype: int = GDN_BF16

    @property
    def D(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.in_dtype == GDN_BF16 else torch.float32

    def c(self) -> _CParams:
        return _CParams(self.num_k_heads, self.num_v_heads, self.head_k_dim, self.head_v_dim,
                        self.conv_kernel, int(self.use_qk_l2norm), self.l2norm_eps, self.in_dtype)


class _CFusion(ctypes.Structure):
    _fields_ = [("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float)]


@dataclasses.dataclass
class GdnFusion:
    """gdn_fusion: optional gate/beta prologue (A_log, dt_bias [Hv]) and gated-RMSNorm
    epilogue (z shaped like o, norm_weight [dv]); tensors in the params' input dtype."""
    A_log: torch.Tensor | None = None
    dt_bias: torch.Tensor | None = None
    z: torch.Tensor | None = None
    norm_weight: torch.Tensor | None = None
    norm_eps: float = 1e-6

    def c(self, p: "GdnParams") -> _CFusion:
        for t, n in ((self.A_log, "A_log"), (self.dt_bias, "dt_bias"), (self.z, "z"),
                     (self.norm_weight, "norm_weight")):
            _expect(t, p.torch_dtype, n)
        return _CFusion(_ptr(self.A_log), _ptr(self.dt_bias), _ptr(self.z), _ptr(self.norm_weight),
                        float(self.norm_eps))


def _fusion_ref(p, fusion):
    return None if fusion is None else ctypes.byref(fusion.c(p))


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m linear_attention_sequence_amd.build`")
    lib = ctypes.CDLL(p)
    V, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    PP = ctypes.POINTER(_CParams)
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = I32
    lib.gdn_conv1d_silu.argtypes = [PP, I32, I32, V, V, V, V, V, V, I32, V]
    lib.gdn_decode_step.argtypes = [PP, I32, V, V, V, V, V, V, V, V, V]
    lib.gdn_verify_block.argtypes = [PP, I32, I32, V, V, V, V, V, V, V, V, V]
    lib.gdn_verify_commit.argtypes = [PP, I32, I32, V, V, V, V, V, V, V]
    lib.gdn_prefill_workspace_size.argtypes = [PP, I32, I32, I32, I32]
    lib.gdn_prefill_workspace_size.restype = SZ
    lib.gdn_prefill.argtypes = [PP, I32, I32, V, V, V, V, V, V, V, V, V, I32, I32, V, SZ, V]
    PF = ctypes.POINTER(_CFusion)
    lib.gdn_decode_step_ex.argtypes = [PP, PF, I32, V, V, V, V, V, V, V, V, V]
    lib.gdn_verify_block_ex.argtypes = [PP, PF, I32, I32, V, V, V, V, V, V, V, V, V]
    lib.gdn_prefill_ex.argtypes = [PP, PF, I32, I32, V, V, V, V, V, V, V, V, V, I32, I32, V, SZ, V]
    lib.gdn_verify_block_slots.argtypes = [PP, PF, I32, I32, V, V, V, V, V, V, I32, V, V, V, V]
    lib.gdn_prefill_ex_noalloc.argtypes = [PP, PF, I32, I32, V, V, V, V, V, V, V, V, V, I32, I32, V]
    for fn in ("gdn_conv1d_silu", "gdn_decode_step", "gdn_verify_block", "gdn_verify_commit",
               "gdn_prefill", "gdn_decode_step_ex", "gdn_verify_block_ex", "gdn_prefill_ex",
               "gdn_verify_block_slots", "gdn_prefill_ex_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _shape(t, expected, name):
    """Raise ValueError unless tensor t (if given) has exactly the shape the call derives
    for it, so that no undersized buffer reaches a kernel."""
    if t is not None and tuple(t.shape) != tuple(expected):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; this call needs {tuple(expected)}")


def _fusion_shapes(p: "GdnParams", fusion, z_shape):
    if fusion is None:
        return
    _shape(fusion.A_log, (p.num_v_heads,), "A_log")
    _shape(fusion.dt_bias, (p.num_v_heads,), "dt_bias")
    _shape(fusion.z, z_shape, "z")
    _shape(fusion.norm_weight, (p.head_v_dim,), "norm_weight")


def _dims(t, n, name):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _call(fn, *args):
    lib = load()
    st = getattr(lib, fn)(*args)
    if st != 0:
        raise GdnError(fn, st, lib.gdn_status_string(st).decode())


def _recurrent_shapes(p, B, T, qkv, gate, beta, conv_weight, conv_state_in, S, o):
    """Shapes shared by the decode and verify calls (T tokens per sequence)."""
    Hv = p.num_v_heads
    _shape(qkv, (B, p.D, T), "qkv")
    _shape(gate, (B, T, Hv), "gate")
    _shape(beta, (B, T, Hv), "beta")
    _shape(conv_weight, (p.D, 1, p.conv_kernel), "conv_weight")
    _shape(conv_state_in, (B, p.D, p.conv_kernel - 1), "conv_state_in")
    _shape(S, (B, Hv, p.head_k_dim, p.head_v_dim), "S")
    _shape(o, (B, T, Hv, p.head_v_dim), "o")


def _prefill_shapes(p, B, L, N, qkv, gate, beta, conv_weight, conv_state_in, conv_state_out, S, o,
                    cu_seqlens):
    Hv, win = p.num_v_heads, (N, p.D, p.conv_kernel - 1)
    _shape(qkv, (B, p.D, L), "qkv")
    _shape(gate, (B, L, Hv), "gate")
    _shape(beta, (B, L, Hv), "beta")
    _shape(conv_weight, (p.D, 1, p.conv_kernel), "conv_weight")
    _shape(conv_state_in, win, "conv_state_in")
    _shape(conv_state_out, win, "conv_state_out")
    _shape(S, (N, Hv, p.head_k_dim, p.head_v_dim), "S")
    _shape(o, (B, L, Hv, p.head_v_dim), "o")
    _shape(cu_seqlens, (N + 1,), "cu_seqlens")


def gdn_version() -> int:
    return int(load().gdn_version())


def gdn_conv1d_silu(p: GdnParams, qkv, conv_weight, conv_state_in, conv_state_out, y,
                    cu_seqlens=None, stream=None):
    """Step 1 alone. qkv [B,D,L]; conv_state_in/out [N,D,K-1]; y [B,D,L] fp32."""
    for t, n in ((qkv, "qkv"), (conv_weight, "conv_weight"), (conv_state_in, "conv_state_in"),
                 (conv_state_out, "conv_state_out")):
        _expect(t, p.torch_dtype, n)
    _expect(y, torch.float32, "y")
    _expect(cu_seqlens, torch.int32, "cu_seqlens")
    B, _, L = _dims(qkv, 3, "qkv")
    N = _dims(conv_state_in, 3, "conv_state_in")[0]
    D, K = p.D, p.conv_kernel
    _shape(qkv, (B, D, L), "qkv")
    _shape(conv_weight, (D, 1, K), "conv_weight")
    _shape(conv_state_in, (N, D, K - 1), "conv_state_in")
    _shape(conv_state_out, (N, D, K - 1), "conv_state_out")
    _shape(y, (B, D, L), "y")
    _shape(cu_seqlens, (N + 1,), "cu_seqlens")
    _call("gdn_conv1d_silu", ctypes.byref(p.c()), B, L, _ptr(qkv), _ptr(conv_weight),
          _ptr(conv_state_in), _ptr(conv_state_out), _ptr(y), _ptr(cu_seqlens), N, _stream(stream))


def gdn_decode_step(p: GdnParams, qkv, gate, beta, conv_weight, conv_state_in, conv_state_out,
                    S, o, stream=None):
    """One token per sequence. qkv [B,D,1]; gate/beta [B,1,Hv]; S [B,Hv,dk,dv] (in place); o [B,1,Hv,dv]."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        _expect(t, p.torch_dtype, n)
    _expect(S, torch.float32, "S")
    _expect(o, torch.float32, "o")
    B = _dims(qkv, 3, "qkv")[0]
    _recurrent_shapes(p, B, 1, qkv, gate, beta, conv_weight, conv_state_in, S, o)
    _shape(conv_state_out, (B, p.D, p.conv_kernel - 1), "conv_state_out")
    _call("gdn_decode_step", ctypes.byref(p.c()), B, _ptr(qkv), _ptr(gate), _ptr(beta),
          _ptr(conv_weight), _ptr(conv_state_in), _ptr(conv_state_out), _ptr(S), _ptr(o),
          _stream(stream))


def gdn_decode_step_ex(p: GdnParams, fusion: GdnFusion | None, qkv, gate, beta, conv_weight,
                       conv_state_in, conv_state_out, S, o, stream=None):
    """gdn_decode_step with the gdn_fusion prologue/epilogue (gate/beta hold raw a/b with A_log)."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        _expect(t, p.torch_dtype, n)
    _expect(S, torch.float32, "S")
    _expect(o, torch.float32, "o")
    B = _dims(qkv, 3, "qkv")[0]
    _recurrent_shapes(p, B, 1, qkv, gate, beta, conv_weight, conv_state_in, S, o)
    _shape(conv_state_out, (B, p.D, p.conv_kernel - 1), "conv_state_out")
    _fusion_shapes(p, fusion, (B, 1, p.num_v_heads, p.head_v_dim))
    _call("gdn_decode_step_ex", ctypes.byref(p.c()), _fusion_ref(p, fusion), B, _ptr(qkv),
          _ptr(gate), _ptr(beta), _ptr(conv_weight), _ptr(conv_state_in), _ptr(conv_state_out),
          _ptr(S), _ptr(o), _stream(stream))


def gdn_verify_block(p: GdnParams, qkv, gate, beta, conv_weight, conv_state_in, S_in, S_snap, o,
                     stream=None):
    """T tokens per sequence with a state snapshot after each. qkv [B,D,T]; S_snap [B,T,Hv,dk,dv]."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in")):
        _expect(t, p.torch_dtype, n)
    for t, n in ((S_in, "S_in"), (S_snap, "S_snap"), (o, "o")):
        _expect(t, torch.float32, n)
    B, _, T = _dims(qkv, 3, "qkv")
    _recurrent_shapes(p, B, T, qkv, gate, beta, conv_weight, conv_state_in, None, o)
    _shape(S_snap, (B, T, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_snap")
    _shape(S_in, (B, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_in")
    _call("gdn_verify_block", ctypes.byref(p.c()), B, T, _ptr(qkv), _ptr(gate), _ptr(beta),
          _ptr(conv_weight), _ptr(conv_state_in), _ptr(S_in), _ptr(S_snap), _ptr(o),
          _stream(stream))


def gdn_verify_block_ex(p: GdnParams, fusion: GdnFusion | None, qkv, gate, beta, conv_weight,
                        conv_state_in, S_in, S_snap, o, stream=None):
    """gdn_verify_block with the gdn_fusion prologue/epilogue."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in")):
        _expect(t, p.torch_dtype, n)
    for t, n in ((S_in, "S_in"), (S_snap, "S_snap"), (o, "o")):
        _expect(t, torch.float32, n)
    B, _, T = _dims(qkv, 3, "qkv")
    _recurrent_shapes(p, B, T, qkv, gate, beta, conv_weight, conv_state_in, None, o)
    _shape(S_snap, (B, T, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_snap")
    _shape(S_in, (B, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_in")
    _fusion_shapes(p, fusion, (B, T, p.num_v_heads, p.head_v_dim))
    _call("gdn_verify_block_ex", ctypes.byref(p.c()), _fusion_ref(p, fusion), B, T, _ptr(qkv),
          _ptr(gate), _ptr(beta), _ptr(conv_weight), _ptr(conv_state_in), _ptr(S_in),
          _ptr(S_snap), _ptr(o), _stream(stream))


def gdn_verify_block_slots(p: GdnParams, fusion: GdnFusion | None, qkv, gate, beta, conv_weight,
                           conv_state_in, S_prev, slot, S_snap, o, stream=None):
    """Verify block starting from snapshot slot[b] of S_prev [B,T_prev,Hv,dk,dv] (may be S_snap)."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in")):
        _expect(t, p.torch_dtype, n)
    for t, n in ((S_prev, "S_prev"), (S_snap, "S_snap"), (o, "o")):
        _expect(t, torch.float32, n)
    _expect(slot, torch.int32, "slot")
    B, _, T = _dims(qkv, 3, "qkv")
    _recurrent_shapes(p, B, T, qkv, gate, beta, conv_weight, conv_state_in, None, o)
    _shape(S_snap, (B, T, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_snap")
    T_prev = _dims(S_prev, 5, "S_prev")[1]
    _shape(S_prev, (B, T_prev, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_prev")
    _shape(slot, (B,), "slot")
    _fusion_shapes(p, fusion, (B, T, p.num_v_heads, p.head_v_dim))
    _call("gdn_verify_block_slots", ctypes.byref(p.c()), _fusion_ref(p, fusion), B, T, _ptr(qkv),
          _ptr(gate), _ptr(beta), _ptr(conv_weight), _ptr(conv_state_in), _ptr(S_prev),
          S_prev.shape[1], _ptr(slot), _ptr(S_snap), _ptr(o), _stream(stream))


def gdn_verify_commit(p: GdnParams, accept_len, qkv, conv_state_in, S_snap, conv_state_out, S_out,
                      stream=None):
    """Keep snapshot accept_len[b] per row and roll the conv window to match
    (S_snap and S_out both None: the conv window only)."""
    _expect(accept_len, torch.int32, "accept_len")
    for t, n in ((qkv, "qkv"), (conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        _expect(t, p.torch_dtype, n)
    _expect(S_snap, torch.float32, "S_snap")
    _expect(S_out, torch.float32, "S_out")
    B, _, T = _dims(qkv, 3, "qkv")
    win = (B, p.D, p.conv_kernel - 1)
    _shape(accept_len, (B,), "accept_len")
    _shape(qkv, (B, p.D, T), "qkv")
    _shape(conv_state_in, win, "conv_state_in")
    _shape(conv_state_out, win, "conv_state_out")
    _shape(S_snap, (B, T, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_snap")
    _shape(S_out, (B, p.num_v_heads, p.head_k_dim, p.head_v_dim), "S_out")
    _call("gdn_verify_commit", ctypes.byref(p.c()), B, T, _ptr(accept_len), _ptr(qkv),
          _ptr(conv_state_in), _ptr(S_snap), _ptr(conv_state_out), _ptr(S_out), _stream(stream))


def gdn_prefill_workspace_size(p: GdnParams, B: int, L: int, N: int, chunk: int = 64) -> int:
    return int(load().gdn_prefill_workspace_size(ctypes.byref(p.c()), B, L, N, chunk))


def gdn_prefill(p: GdnParams, qkv, gate, beta, conv_weight, conv_state_in, conv_state_out, S, o,
                workspace, cu_seqlens=None, chunk: int = 64, stream=None):
    """A whole prompt (or N packed prompts with cu_seqlens). S [N,Hv,dk,dv] in place; o [B,L,Hv,dv]."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        _expect(t, p.torch_dtype, n)
    _expect(S, torch.float32, "S")
    _expect(o, torch.float32, "o")
    _expect(cu_seqlens, torch.int32, "cu_seqlens")
    B, _, L = _dims(qkv, 3, "qkv")
    N = _dims(S, 4, "S")[0]
    _prefill_shapes(p, B, L, N, qkv, gate, beta, conv_weight, conv_state_in, conv_state_out, S, o, cu_seqlens)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("gdn_prefill", ctypes.byref(p.c()), B, L, _ptr(qkv), _ptr(gate), _ptr(beta),
          _ptr(conv_weight), _ptr(conv_state_in), _ptr(conv_state_out), _ptr(S), _ptr(o),
          _ptr(cu_seqlens), N, chunk, _ptr(workspace), ws_bytes, _stream(stream))


def gdn_prefill_ex(p: GdnParams, fusion: GdnFusion | None, qkv, gate, beta, conv_weight,
                   conv_state_in, conv_state_out, S, o, workspace, cu_seqlens=None, chunk: int = 64,
                   stream=None):
    """gdn_prefill with the gdn_fusion prologue/epilogue."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        _expect(t, p.torch_dtype, n)
    _expect(S, torch.float32, "S")
    _expect(o, torch.float32, "o")
    _expect(cu_seqlens, torch.int32, "cu_seqlens")
    B, _, L = _dims(qkv, 3, "qkv")
    N = _dims(S, 4, "S")[0]
    _prefill_shapes(p, B, L, N, qkv, gate, beta, conv_weight, conv_state_in, conv_state_out, S, o, cu_seqlens)
    _fusion_shapes(p, fusion, (B, L, p.num_v_heads, p.head_v_dim))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("gdn_prefill_ex", ctypes.byref(p.c()), _fusion_ref(p, fusion), B, L, _ptr(qkv),
          _ptr(gate), _ptr(beta), _ptr(conv_weight), _ptr(conv_state_in), _ptr(conv_state_out),
          _ptr(S), _ptr(o), _ptr(cu_seqlens), N, chunk, _ptr(workspace), ws_bytes, _stream(stream))


def gdn_prefill_ex_noalloc(p: GdnParams, fusion: GdnFusion | None, qkv, gate, beta, conv_weight,
                           conv_state_in, conv_state_out, S, o, cu_seqlens=None, chunk: int = 64,
                           stream=None):
    """gdn_prefill_ex with the library's static device scratch as its workspace (no
    allocation: for callers that cannot allocate). Raises GdnError(GDN_ERR_TOO_LARGE) when
    the prompt needs more than the 128 MiB scratch."""
    for t, n in ((qkv, "qkv"), (gate, "gate"), (beta, "beta"), (conv_weight, "conv_weight"),
                 (conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        _expect(t, p.torch_dtype, n)
    _expect(S, torch.float32, "S")
    _expect(o, torch.float32, "o")
    _expect(cu_seqlens, torch.int32, "cu_seqlens")
    B, _, L = _dims(qkv, 3, "qkv")
    N = _dims(S, 4, "S")[0]
    _prefill_shapes(p, B, L, N, qkv, gate, beta, conv_weight, conv_state_in, conv_state_out, S, o, cu_seqlens)
    _fusion_shapes(p, fusion, (B, L, p.num_v_heads, p.head_v_dim))
    _call("gdn_prefill_ex_noalloc", ctypes.byref(p.c()), _fusion_ref(p, fusion), B, L, _ptr(qkv),
          _ptr(gate), _ptr(beta), _ptr(conv_weight), _ptr(conv_state_in), _ptr(conv_state_out),
          _ptr(S), _ptr(o), _ptr(cu_seqlens), N, chunk, _stream(stream))


def prefill_workspace(p: GdnParams, B: int, L: int, N: int, chunk: int = 64, device="cuda"):
    """Allocate a workspace tensor of gdn_prefill_workspace_size() bytes (256-byte aligned)."""
    n = gdn_prefill_workspace_size(p, B, L, N, chunk)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)
