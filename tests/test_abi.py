"""CPU-only checks of the C-ABI library: it loads, exports every symbol the header
declares, and its synchronous validation returns the documented status codes
without launching anything (all calls below fail validation, or have nothing to
do, before any HIP call is made; the pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, DTYPE, UNSUP, ALIAS, WS, LAUNCH, ALIGN, TOO_LARGE = range(10)


def header_symbols(header="gdn.h"):
    with open(os.path.join(ROOT, "include", header)) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(gdn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        from linear_attention_sequence_amd import build
        build.build()
    return gdn.load()


def test_header_lists_the_binding_exports():
    assert header_symbols() == sorted(gdn.EXPORTS)


def test_library_exports_every_header_symbol(lib):
    for name in header_symbols():
        assert hasattr(lib, name), name


def test_ceiling_library_exports_and_validation(lib):
    """The measurement library of include/gdn_ceiling.h loads, exports its calls, and rejects
    bad arguments (status 1) before any launch."""
    path = os.path.join(os.path.dirname(gdn.LIB_PATH), "libgdn_ceiling.so")
    assert os.path.exists(path)
    cl = ctypes.CDLL(path)
    names = header_symbols("gdn_ceiling.h")
    assert names == ["gdn_ceiling_copy", "gdn_ceiling_copy_blocked", "gdn_ceiling_device_info",
                     "gdn_ceiling_mfma", "gdn_ceiling_read", "gdn_ceiling_read_blocked", "gdn_ceiling_write",
                     "gdn_ceiling_write_blocked"]
    for name in names:
        assert hasattr(cl, name), name
    V, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    cl.gdn_ceiling_copy.argtypes = [V, V, SZ, I, I, V]
    cl.gdn_ceiling_mfma.argtypes = [V, I, I, I, V]
    cl.gdn_ceiling_read.argtypes = [V, SZ, V, I, V]
    assert cl.gdn_ceiling_copy(A(1), A(1), 1 << 20, 1, 1024, None) == 1           # overlap
    assert cl.gdn_ceiling_copy(A(1), A(2), 100, 1, 1024, None) == 1               # not a multiple of 64
    assert cl.gdn_ceiling_read(A(1), 1 << 20, A(2), 0, None) == 1                 # empty grid
    assert cl.gdn_ceiling_mfma(A(1), 256, 10, 4, None) == 1                       # unknown dtype
    cl.gdn_ceiling_copy_blocked.argtypes = [V, V, SZ, I, I, V]
    cl.gdn_ceiling_read_blocked.argtypes = [V, SZ, V, I, V]
    cl.gdn_ceiling_write_blocked.argtypes = [V, SZ, I, I, V]
    assert cl.gdn_ceiling_copy_blocked(A(1), A(2), 1 << 20, 1, 5, None) == 1      # per_thread not 4, 8, 16
    assert cl.gdn_ceiling_copy_blocked(A(1), A(2), 3 << 12, 1, 4, None) == 1      # not a multiple of the 16 KB block
    assert cl.gdn_ceiling_copy_blocked(A(1), A(1), 1 << 20, 1, 16, None) == 1     # overlap
    assert cl.gdn_ceiling_read_blocked(A(1), 1 << 20, None, 8, None) == 1         # no sink
    assert cl.gdn_ceiling_write_blocked(A(1), 1 << 40, 1, 4, None) == 1           # more than 2^20 blocks


def test_status_strings_and_version(lib):
    for code in range(10):
        assert lib.gdn_status_string(code)
    assert lib.gdn_version() >= 10000


def P(**kw):
    d = dict(num_k_heads=16, num_v_heads=32, head_k_dim=128, head_v_dim=128, conv_kernel=4,
             use_qk_l2norm=True, l2norm_eps=1e-6, in_dtype=gdn.GDN_BF16)
    d.update(kw)
    return ctypes.byref(gdn.GdnParams(**d).c())


# fake, well-separated, 256-byte aligned device addresses: never dereferenced
def A(i):
    return ctypes.c_void_p(0x7f0000000000 + i * 0x100000000)


def decode(lib, p, B=4, **over):
    args = dict(qkv=A(1), gate=A(2), beta=A(3), w=A(4), cin=A(5), cout=A(6), S=A(7), o=A(8))
    args.update(over)
    return lib.gdn_decode_step(p, B, args["qkv"], args["gate"], args["beta"], args["w"],
                               args["cin"], args["cout"], args["S"], args["o"], None)


def test_param_validation(lib):
    assert decode(lib, None) == NULL
    assert decode(lib, P(in_dtype=7)) == DTYPE
    assert decode(lib, P(num_k_heads=0)) == SHAPE
    assert decode(lib, P(num_k_heads=3, num_v_heads=32)) == SHAPE      # Hv % Hk != 0
    assert decode(lib, P(use_qk_l2norm=2)) == SHAPE
    assert decode(lib, P(l2norm_eps=-1.0)) == SHAPE
    assert decode(lib, P(l2norm_eps=float("nan"))) == SHAPE
    assert decode(lib, P(head_k_dim=32, head_v_dim=32)) == UNSUP
    assert decode(lib, P(head_k_dim=256, head_v_dim=256)) == UNSUP
    assert decode(lib, P(head_k_dim=128, head_v_dim=16)) == UNSUP
    assert decode(lib, P(conv_kernel=3)) == UNSUP


def test_decode_validation(lib):
    p = P()
    assert decode(lib, p, B=-1) == SHAPE
    assert decode(lib, p, B=0) == OK                  # nothing to do, nothing launched
    for k in ("qkv", "gate", "beta", "w", "cin", "cout", "S", "o"):
        assert decode(lib, p, **{k: None}) == NULL, k
    assert decode(lib, p, cout=A(5)) == ALIAS          # conv_state_out == conv_state_in
    assert decode(lib, p, o=A(7)) == ALIAS             # o inside S
    assert decode(lib, p, S=ctypes.c_void_p(0x7f0000000004)) == ALIGN


def test_verify_and_commit_validation(lib):
    p = P()

    def verify(B=4, T=4, S_in=A(7), S_snap=A(9), o=A(8)):
        return lib.gdn_verify_block(p, B, T, A(1), A(2), A(3), A(4), A(5), S_in, S_snap, o, None)

    assert verify(T=0) == SHAPE
    assert verify(T=17) == UNSUP
    assert verify(S_in=None) == NULL
    assert verify(S_snap=A(7)) == ALIAS
    assert verify(B=0) == OK

    def commit(B=4, T=4, acc=A(10), cin=A(5), snap=A(9), cout=A(6), S_out=A(7)):
        return lib.gdn_verify_commit(p, B, T, acc, A(1), cin, snap, cout, S_out, None)

    assert commit(T=0) == SHAPE
    assert commit(acc=None) == NULL
    assert commit(cout=A(5)) == ALIAS
    assert commit(S_out=A(9)) == ALIAS
    assert commit(B=0) == OK


def test_conv_validation(lib):
    p = P()

    def conv(B=2, L=8, cu=None, N=2, cin=A(5), cout=A(6), y=A(8)):
        return lib.gdn_conv1d_silu(p, B, L, A(1), A(4), cin, cout, y, cu, N, None)

    assert conv(N=3) == SHAPE                  # without cu_seqlens N must equal B
    assert conv(cu=A(11), B=2) == SHAPE        # with cu_seqlens B must be 1
    assert conv(L=-1) == SHAPE
    assert conv(y=None) == NULL
    assert conv(cout=A(5)) == ALIAS
    assert conv(B=0, N=0) == OK


def test_prefill_validation(lib):
    p = P()
    need = lib.gdn_prefill_workspace_size(p, 1, 4096, 1, 64)
    assert need > 0
    assert lib.gdn_prefill_workspace_size(p, 1, 4096, 1, 32) == 0   # chunk 32 unsupported
    assert lib.gdn_prefill_workspace_size(None, 1, 4096, 1, 64) == 0

    def prefill(B=1, L=4096, N=1, cu=None, chunk=64, ws=A(12), ws_bytes=need, S=A(7), o=A(8)):
        return lib.gdn_prefill(p, B, L, A(1), A(2), A(3), A(4), A(5), A(6), S, o, cu, N, chunk,
                               ws, ws_bytes, None)

    assert prefill(chunk=32) == UNSUP
    assert prefill(chunk=0) == SHAPE
    assert prefill(N=2) == SHAPE
    assert prefill(ws=None) == WS
    assert prefill(ws_bytes=1) == WS
    assert prefill(ws=ctypes.c_void_p(0x7f0000000010 + 12 * 0x100000000)) == ALIGN
    assert prefill(o=A(7)) == ALIAS
    assert prefill(ws=A(8)) == ALIAS
    assert prefill(B=2, N=2, cu=A(11)) == SHAPE
    # the bound for (B = 1, L, N = 1) serves the call unpacked or through cu_seqlens, with or
    # without the gated RMSNorm: it is the need of the largest of those layouts (unpacked
    # with the norm, whose carry runs in more segments), one byte less is refused for that
    # call and is still enough for the others
    def fused(ws_bytes):
        return lib.gdn_prefill_ex(p, F(z=A(13), w=A(14)), 1, 4096, A(1), A(2), A(3), A(4), A(5), A(6), A(7),
                                  A(8), None, 1, 64, A(12), ws_bytes, None)
    assert fused(need - 1) == WS
    assert fused(need) != WS
    assert prefill(ws_bytes=need - 1) != WS
    assert prefill(N=1, cu=A(11), ws_bytes=need - 1) != WS
    assert lib.gdn_prefill_workspace_size(p, 1, 4096, 8, 64) > 0
    assert prefill(N=0, cu=A(11)) == OK


def F(A_log=None, dt_bias=None, z=None, w=None, eps=1e-6):
    return ctypes.byref(gdn._CFusion(A_log, dt_bias, z, w, eps))


def test_fusion_validation(lib):
    p = P()

    def dec(fu, B=4, o=A(8)):
        return lib.gdn_decode_step_ex(p, fu, B, A(1), A(2), A(3), A(4), A(5), A(6), A(7), o, None)

    def ver(fu, B=4, T=4):
        return lib.gdn_verify_block_ex(p, fu, B, T, A(1), A(2), A(3), A(4), A(5), A(7), A(9),
                                       A(8), None)

    need = lib.gdn_prefill_workspace_size(p, 1, 4096, 1, 64)

    def pre(fu, B=1, L=4096, N=1):
        return lib.gdn_prefill_ex(p, fu, B, L, A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8),
                                  None, N, 64, A(12), need, None)

    for call in (dec, ver, pre):
        assert call(F(A_log=A(13))) == NULL, call            # A_log without dt_bias
        assert call(F(z=A(15))) == NULL, call                # z without norm_weight
        assert call(F(z=A(15), w=A(16), eps=-1.0)) == SHAPE, call
        assert call(F(z=A(15), w=A(16), eps=float("inf"))) == SHAPE, call
        assert call(F(z=A(8), w=A(16))) == ALIAS, call       # z == o
        assert call(F(A_log=A(13), dt_bias=A(8))) == ALIAS, call   # dt_bias == o
    # an empty call is valid with any complete fusion, and NULL fusion is the plain call
    assert dec(F(A_log=A(13), dt_bias=A(14), z=A(15), w=A(16)), B=0) == OK
    assert ver(F(A_log=A(13), dt_bias=A(14)), B=0) == OK
    assert pre(F(z=A(15), w=A(16)), B=0, N=0) == OK
    assert dec(None, B=0) == OK
    # fields of a disabled fusion are ignored (dt_bias without A_log, eps without z)
    assert dec(F(dt_bias=A(8), eps=float("nan")), B=0) == OK


def test_verify_slots_and_window_only_commit_validation(lib):
    p = P()

    def vs(B=4, T=4, S_prev=A(7), T_prev=4, slot=A(10), S_snap=A(9), o=A(8)):
        return lib.gdn_verify_block_slots(p, None, B, T, A(1), A(2), A(3), A(4), A(5), S_prev, T_prev,
                                          slot, S_snap, o, None)

    assert vs(slot=None) == NULL
    assert vs(S_prev=None) == NULL
    assert vs(T_prev=0) == SHAPE
    assert vs(T_prev=17) == UNSUP
    assert vs(S_snap=A(7), T_prev=3) == ALIAS          # same buffer, different block widths
    assert vs(S_snap=ctypes.c_void_p(0x7f0000000000 + 7 * 0x100000000 + 4096), T_prev=4) == ALIAS
    assert vs(slot=A(9)) == ALIAS                        # slot inside the snapshots being written
    assert vs(B=0) == OK
    assert vs(B=0, S_snap=A(7)) == OK                    # in place (T == T_prev)

    def commit(S_snap=A(9), S_out=A(7), cout=A(6)):
        return lib.gdn_verify_commit(p, 4, 4, A(10), A(1), A(5), S_snap, cout, S_out, None)

    assert commit(S_snap=None) == NULL                   # one of the two only
    assert commit(S_out=None) == NULL
    assert commit(S_snap=None, S_out=None, cout=A(5)) == ALIAS


def test_noalloc_prefill_rejects_prompts_beyond_its_scratch(lib):
    """gdn_prefill_ex_noalloc checks the need against its 128 MiB static scratch before it
    touches the GPU: an 8192-token prompt at 16/32 heads needs more and is refused."""
    p = P()
    need = lib.gdn_prefill_workspace_size(p, 1, 8192, 1, 64)
    assert need > (128 << 20)
    st = lib.gdn_prefill_ex_noalloc(p, None, 1, 8192, A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8),
                                    None, 1, 64, None)
    assert st == TOO_LARGE
    assert b"static scratch" in lib.gdn_status_string(TOO_LARGE)
    # invalid arguments are reported as gdn_prefill_ex reports them (need is 0 for them)
    assert lib.gdn_prefill_ex_noalloc(p, None, 1, 64, A(1), A(2), A(3), A(4), A(5), A(6), A(7), A(8),
                                      None, 1, 32, None) == UNSUP
